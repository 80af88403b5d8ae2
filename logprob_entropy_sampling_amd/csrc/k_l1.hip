// Draft/target softmax L1 distance (DeepSpec PR #87, Purpose: the per-token
// distance sum_v |P_v - Q_v| computed once and shared by
// accept_rate = clamp(1 - 0.5 * L1, 0, 1) and the L1 loss).
//
// Two kernels.  l1_kernel (any dtype, any row length): one workgroup per
// token row; pass 1 streams both rows once and folds each into an online
// (max, sum-exp) state; pass 2 streams them again and sums
// |2^(u - M - log2 S) - 2^(w - M' - log2 S')|, the normalisers folded into the
// exponent so each probability is one FMA + one v_exp_f32.
// l1_resident_kernel (bf16 rows of 65,537 to 155,655 logits): one workgroup
// per CU keeps one row of each pair in registers and half of the other in
// LDS, so HBM is read 1.25 times instead of twice (described below).
// No probability vector is stored anywhere.  Identical rows give exactly 0:
// both sides run the same instructions on the same bits.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "../../include/vocabscore.h"

namespace vs {

namespace {


struct Pair {
  float mx, sx, my, sy;
};

// Online (max, sum 2^((x - max) log2 e)) update with a block of raw logits.
// m is kept in raw units (the max is taken on the logits themselves); each
// term is one FMA and one v_exp_f32.  No floor is needed: there is no
// e * d term, exp2(-inf) = 0, and a NaN poisons s as it should.
__device__ __forceinline__ void online(float& m, float& s, const float* v, int n, float l2e) {
  float bm = v[0];
  for (int i = 1; i < n; ++i) bm = fmaxf(bm, v[i]);
  const float nm = fmaxf(m, bm);
  if (nm == kNegInf) {  // only -inf so far, or a NaN that fmaxf dropped
    for (int i = 0; i < n; ++i)
      if (v[i] != v[i]) s = __builtin_nanf("");
    return;
  }
  const float c = nm * l2e;
  s *= exp2_hw(m * l2e - c);  // exactly 1 when the max did not move; 0 from -inf
  for (int i = 0; i < n; ++i) s += exp2_hw(__builtin_fmaf(v[i], l2e, -c));
  m = nm;
}

// raw values of element chunk q (VEC elements) of a row.  Streaming loads in
// both passes: a row pair (607 KB at V = 151,936) does not stay in L2 until
// the second pass, and plain loads cap the reads near 5.4 TB/s.
template <int DT>
__device__ __forceinline__ void load_chunk(const void* row, int64_t q, float* v) {
  if (DT == VS_BF16) {
    const uint4* pw = reinterpret_cast<const uint4*>(row) + q;
    const uint4 w = stream_load(pw);
    v[0] = bf16_lo(w.x);
    v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y);
    v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z);
    v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w);
    v[7] = bf16_hi(w.w);
  } else {
    const float4* pw = reinterpret_cast<const float4*>(row) + q;
    const float4 w = stream_load(pw);
    v[0] = w.x;
    v[1] = w.y;
    v[2] = w.z;
    v[3] = w.w;
  }
}

template <int DT>
__device__ __forceinline__ float load_one(const void* row, int64_t i) {
  return DT == VS_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(row)[i]) : static_cast<const float*>(row)[i];
}

// A row's base-2 normaliser: p_v = 2^(u_v - m - l2s), l2s = log2 of the sum
// against the maximum m.  The fast form subtracts l = m + l2s in the same FMA
// as the scale; once |m| reaches 2^13 the rounding of l (up to 2^-12 in the
// exponent, the same for every element of the row) would show, and the
// accurate form subtracts m and l2s one after the other (one more operation
// per element, on such rows only).
struct Norm {
  float m, l2s, l;
};
constexpr float kBigRef = 0x1p13f;
// l1 marker of a row the resident kernel redoes in the accurate form after its row loop (no L1 is negative)
constexpr float kL1Redo = -1.0f;

__device__ __forceinline__ Norm make_norm(float m, float s) {
  const float l2s = log2_hw(s);
  return Norm{m, l2s, m + l2s};
}
__device__ __forceinline__ bool norm_ok(const Norm& n) { return n.l > -__builtin_inff() && n.l < __builtin_inff(); }
// row-uniform choice of the accurate form (a scalar value: the branch does not diverge)
__device__ __forceinline__ bool norms_big(const Norm& x, const Norm& y) {
  return __builtin_amdgcn_readfirstlane(int(!(fabsf(x.m) < kBigRef && fabsf(y.m) < kBigRef))) != 0;
}

// |p - q| of one element pair, the normalisers folded into the exponents
template <bool ACC>
__device__ __forceinline__ float absdiff(float a, float b, const Norm& x, const Norm& y, float l2e) {
  if (ACC)
    return fabsf(exp2_hw(__builtin_fmaf(a, l2e, -x.m) - x.l2s) - exp2_hw(__builtin_fmaf(b, l2e, -y.m) - y.l2s));
  return fabsf(exp2_hw(__builtin_fmaf(a, l2e, -x.l)) - exp2_hw(__builtin_fmaf(b, l2e, -y.l)));
}

// One row pair by one workgroup of NT threads, U vector chunks per thread in
// flight per pass step: pass 1 (online max / sum-exp of both rows), merge,
// pass 2 (sum |p - q|).
template <int DT, int NT, int U>
__device__ __forceinline__ void l1_row(const void* __restrict__ tgt, int64_t ld_t, const void* __restrict__ dft,
                                       int64_t ld_d, int64_t V, int64_t row, float* __restrict__ l1,
                                       float* __restrict__ accept) {
  constexpr int VEC = DT == VS_BF16 ? 8 : 4;
  constexpr int ES = DT == VS_BF16 ? 2 : 4;
  constexpr int NW = NT / 64;
  // base-2 scale: log2(e), rounded to 16 bits for bf16 rows (exact products)
  constexpr float l2e = DT == VS_BF16 ? kLog2eBf16 : kLog2e;
  __shared__ float red[NW][4];
  const int tid = threadIdx.x;
  const char* trow = static_cast<const char*>(tgt) + row * ld_t * ES;
  const char* drow = static_cast<const char*>(dft) + row * ld_d * ES;
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(trow) | reinterpret_cast<uintptr_t>(drow)) & 15) == 0;
  const int64_t nvec = vec_ok ? V / VEC : 0;
  const int64_t tail0 = nvec * VEC;

  // ---- pass 1: online max / sum-exp of both rows ----
  float mx = kNegInf, sx = 0.0f, my = kNegInf, sy = 0.0f;
  int64_t q = tid;
  for (; q + int64_t(U - 1) * NT < nvec; q += int64_t(U) * NT) {
    float a[U][VEC], b[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load_chunk<DT>(trow, q + u * NT, a[u]);
      load_chunk<DT>(drow, q + u * NT, b[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      online(mx, sx, a[u], VEC, l2e);
      online(my, sy, b[u], VEC, l2e);
    }
  }
  for (; q < nvec; q += NT) {
    float a[VEC], b[VEC];
    load_chunk<DT>(trow, q, a);
    load_chunk<DT>(drow, q, b);
    online(mx, sx, a, VEC, l2e);
    online(my, sy, b, VEC, l2e);
  }
  for (int64_t i = tail0 + tid; i < V; i += NT) {
    float a = load_one<DT>(trow, i), b = load_one<DT>(drow, i);
    online(mx, sx, &a, 1, l2e);
    online(my, sy, &b, 1, l2e);
  }
  // block merge (fixed tree): wave tree, then wave 0 over the NW wave states;
  // the merge works in base-2 units
  Part px = wave_merge_to_lane0(Part{mx * l2e, sx, 0.0f});
  Part py = wave_merge_to_lane0(Part{my * l2e, sy, 0.0f});
  if ((tid & 63) == 0) {
    red[tid >> 6][0] = px.m;
    red[tid >> 6][1] = px.s;
    red[tid >> 6][2] = py.m;
    red[tid >> 6][3] = py.s;
  }
  __syncthreads();
  __shared__ float fin[4];
  if (tid < 64) {
    Part qx{kNegInf, 0.0f, 0.0f}, qy{kNegInf, 0.0f, 0.0f};
    if (tid < NW) {
      qx = Part{red[tid][0], red[tid][1], 0.0f};
      qy = Part{red[tid][2], red[tid][3], 0.0f};
    }
    qx = wave_merge_to_lane0(qx);
    qy = wave_merge_to_lane0(qy);
    if (tid == 0) {
      fin[0] = qx.m;  // base-2 maximum and sum of the target row
      fin[1] = qx.s;
      fin[2] = qy.m;
      fin[3] = qy.s;
    }
  }
  __syncthreads();
  const Norm nx = make_norm(fin[0], fin[1]), ny = make_norm(fin[2], fin[3]);
  const bool ok = norm_ok(nx) && norm_ok(ny);
  if (!ok) {
    if (tid == 0) {
      l1[row] = __builtin_nanf("");
      if (accept) accept[row] = __builtin_nanf("");
    }
    return;
  }

  // ---- pass 2: sum |p - q| ----
  auto pass2 = [&](auto acc_form) {
    constexpr bool ACC = decltype(acc_form)::value;
    float acc = 0.0f;
    int64_t q = tid;
    for (; q + int64_t(U - 1) * NT < nvec; q += int64_t(U) * NT) {
      float a[U][VEC], b[U][VEC];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        load_chunk<DT>(trow, q + u * NT, a[u]);
        load_chunk<DT>(drow, q + u * NT, b[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc += absdiff<ACC>(a[u][i], b[u][i], nx, ny, l2e);
    }
    for (; q < nvec; q += NT) {
      float a[VEC], b[VEC];
      load_chunk<DT>(trow, q, a);
      load_chunk<DT>(drow, q, b);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc += absdiff<ACC>(a[i], b[i], nx, ny, l2e);
    }
    for (int64_t i = tail0 + tid; i < V; i += NT) {
      const float a = load_one<DT>(trow, i), b = load_one<DT>(drow, i);
      acc += absdiff<ACC>(a, b, nx, ny, l2e);
    }
    return acc;
  };
  float acc = norms_big(nx, ny) ? pass2(std::true_type{}) : pass2(std::false_type{});
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = shfl_down_f(acc, off);
    if ((tid & ((off << 1) - 1)) == 0) acc += o;
  }
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6][0] = acc;
  __syncthreads();
  if (tid < 64) {
    float v = tid < NW ? red[tid][0] : 0.0f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = shfl_down_f(v, off);
      if ((tid & ((off << 1) - 1)) == 0) v += o;
    }
    if (tid == 0) {
      const float d = fminf(fmaxf(v, 0.0f), 2.0f);
      l1[row] = d;
      if (accept) accept[row] = fminf(fmaxf(1.0f - 0.5f * d, 0.0f), 1.0f);
    }
  }
}

template <int DT, int NT, int U>
__global__ __launch_bounds__(NT) void l1_kernel(const void* __restrict__ tgt, int64_t ld_t, const void* __restrict__ dft,
                                                int64_t ld_d, int64_t V, float* __restrict__ l1,
                                                float* __restrict__ accept) {
  l1_row<DT, NT, U>(tgt, ld_t, dft, ld_d, V, blockIdx.x, l1, accept);
}

// ---------------------------------------------------------------------------
// Resident form (bf16 rows, 65,536 < V <= 155,655, 16-byte aligned rows).
//
// A row pair (2 x V x 2 bytes, 607 KB at V = 151,936) does not fit one CU's
// registers and LDS together, but one row and half of the other do.  One
// 512-thread workgroup per CU walks rows blockIdx.x, blockIdx.x + gridDim.x, ...
//   * the draft row lives in VGPRs: thread t holds 16-byte chunks
//     t + 512 j, j < 38 (152 registers);
//   * pass 1 streams the target row once, sums both rows' exponentials
//     against per-thread references that move only on overflow (no per-chunk
//     maximum or rescale), and keeps target chunks j < 19 in LDS;
//   * the wave and workgroup merges run once per row behind one barrier:
//     each wave writes its merged state to LDS and every wave combines the
//     eight states itself, in the same order; the pass-2 partial sums are
//     added up by thread 0 after the next row's barrier (LDS partials are
//     double-buffered by row parity);
//   * pass 2 takes those chunks from LDS, re-reads target chunks j >= 19
//     (about a quarter of the pair's bytes) and, as soon as draft chunk j
//     has been used, loads the next row's draft chunk j into the same
//     registers, so the next row's draft arrives during this row's pass 2.
// HBM reads per row pair: 1.25x the pair's bytes, against 2x for the
// two-pass kernel above.  Loads are buffer loads against a per-row resource
// of nvec x 16 bytes: a chunk past the row's last full chunk, or any chunk of
// a row that does not exist (no next row), reads 0 without touching memory,
// and is never used.  The < 8 tail elements of a row are read one per
// thread.  Both rows of a pair run the same instructions in the same order,
// so identical rows still give exactly 0.
// Measured at T = 2048, V = 151,936: about 261 us against 356 us for the
// two-pass kernel; about 71k shader cycles per row per CU, of which the VALU
// work is about 48k.  Tried and not kept: sending the LDS half by
// buffer-to-LDS loads at the start of pass 1 (the streamed chunks then wait
// behind them), or refilling each LDS slot for the next row during pass 2
// (pass 2 slows by more than pass 1 gains).
// ---------------------------------------------------------------------------
constexpr int RES_NT = 512;  // threads per workgroup (8 waves, 2 per SIMD: up to 256 VGPRs each)
constexpr int RES_JD = 38;   // draft chunks per thread, in VGPRs
constexpr int RES_JL = 19;   // target chunks per thread kept in LDS (19 x 8 KiB = 152 KiB)
constexpr int RES_U = 4;     // streamed target chunks in flight per thread
constexpr int64_t kResMaxVec = int64_t(RES_JD) * RES_NT;  // 19,456 chunks of 8 logits
constexpr int64_t kResMinV = 65537;
constexpr int kBufFlags = 0x00020000;  // dword 3 of a raw buffer resource: 32-bit data format
constexpr int kNtAux = 2;              // buffer-load cache policy bit: non-temporal


__device__ __forceinline__ uint4 res_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, int j) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, j * RES_NT * 16, kNtAux);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void unpack8(const uint4& w, float* v) {
  v[0] = bf16_lo(w.x);
  v[1] = bf16_hi(w.x);
  v[2] = bf16_lo(w.y);
  v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z);
  v[5] = bf16_hi(w.z);
  v[6] = bf16_lo(w.w);
  v[7] = bf16_hi(w.w);
}

// s += sum_i 2^(v_i log2 e - c) against a reference c (base-2 units) that
// moves only when it must: a chunk whose sum is not below 2^64 (a term far
// above c, the initial c = -inf, or a NaN) is summed again after c moves to
// the chunk's largest logit.  No per-chunk maximum or rescale otherwise;
// terms stay below 2^64 each, so s cannot overflow for any row length here.
template <int N>
__device__ __forceinline__ void lazy_add(float& c, float& s, const float* v) {
  float cs = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) cs += exp2_hw(__builtin_fmaf(v[i], kLog2eBf16, -c));
  if (!(cs < 0x1p64f)) {
    float bm = v[0];
#pragma unroll
    for (int i = 1; i < N; ++i) bm = fmaxf(bm, v[i]);
    const float nc = fmaxf(c, bm * kLog2eBf16);
    cs = 0.0f;
    if (nc == kNegInf) {  // only -inf so far (or NaNs that fmaxf dropped)
#pragma unroll
      for (int i = 0; i < N; ++i)
        if (v[i] != v[i]) cs = __builtin_nanf("");
    } else {
      s *= exp2_hw(c - nc);  // 0 from the initial -inf
      c = nc;
#pragma unroll
      for (int i = 0; i < N; ++i) cs += exp2_hw(__builtin_fmaf(v[i], kLog2eBf16, -c));
    }
  }
  s += cs;
}

// weight of a state with reference c inside a merge whose reference is M >= c
__device__ __forceinline__ float ref_scale(float c, float M) { return c == M ? 1.0f : exp2_hw(c - M); }

// Wave maximum and sum with DPP moves (no LDS round trips): shifts by 1, 2,
// 4, 8 inside each row of 16 lanes, then lane 15 of rows 0 and 2 into rows 1
// and 3, then lane 31 into rows 2 and 3; lanes with no source take the
// operation's identity.  Lane 63 ends with the result, read into a scalar
// register.  A fixed order, so the sums are reproducible.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float v, float identity) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
template <class Op>
__device__ __forceinline__ float wave_reduce(float x, float identity, Op op) {
  x = op(x, dpp_f32<0x111, 0xf>(x, identity));  // row_shr:1
  x = op(x, dpp_f32<0x112, 0xf>(x, identity));  // row_shr:2
  x = op(x, dpp_f32<0x114, 0xf>(x, identity));  // row_shr:4
  x = op(x, dpp_f32<0x118, 0xf>(x, identity));  // row_shr:8
  x = op(x, dpp_f32<0x142, 0xa>(x, identity));  // row_bcast:15 into rows 1, 3
  x = op(x, dpp_f32<0x143, 0xc>(x, identity));  // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float wave_max_all(float v) {
  return wave_reduce(v, kNegInf, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum_all(float v) {
  return wave_reduce(v, 0.0f, [](float a, float b) { return a + b; });
}

__global__ __launch_bounds__(RES_NT) void l1_resident_kernel(const uint16_t* __restrict__ tgt, int64_t ld_t,
                                                             const uint16_t* __restrict__ dft, int64_t ld_d,
                                                             int64_t rows, int64_t V, float* __restrict__ l1,
                                                             float* __restrict__ accept) {
  constexpr int NW = RES_NT / 64;
  __shared__ uint4 keep[RES_JL][RES_NT];
  // per-wave partials, double-buffered by row parity: one barrier per row
  // orders every write after the reads of the same buffer two rows earlier
  __shared__ float red_a[2][NW][4];  // pass 1: (c, s) of both rows
  __shared__ float red_b[2][NW];     // pass 2: sum |p - q|
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t nvec = V >> 3;
  const int ntail = int(V - nvec * 8);
  const uint32_t voff = uint32_t(tid) * 16;
  const int nj = tid < nvec ? int((nvec - 1 - tid) / RES_NT) + 1 : 0;  // this thread's chunks
  const int nbytes = int(nvec * 16);
  auto rsrc = [&](const uint16_t* base, int64_t ld, int64_t r) {
    const bool live = r < rows;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (live ? r : 0) * ld), (short)0, live ? nbytes : 0,
                                             kBufFlags);
  };
  // row r's L1 from the pass-2 partials of buffer b (thread 0); state 0: a
  // non-finite normaliser (NaN), 1: done, 2: the maxima need the accurate
  // form, redone after the row loop (the kL1Redo marker until then)
  auto finish = [&](int64_t r, int b, int state) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red_b[b][w];
    const float nan = __builtin_nanf("");
    const float dd = state == 1 ? fminf(fmaxf(v, 0.0f), 2.0f) : state == 2 ? kL1Redo : nan;
    l1[r] = dd;
    if (accept) accept[r] = state == 1 ? fminf(fmaxf(1.0f - 0.5f * dd, 0.0f), 1.0f) : nan;
  };

  int64_t row = blockIdx.x;
  uint4 d[RES_JD];
  {
    const __amdgpu_buffer_rsrc_t rd = rsrc(dft, ld_d, row);
#pragma unroll
    for (int j = 0; j < RES_JD; ++j) d[j] = res_load(rd, voff, j);
  }
  int prev_state = 0;
  // rows this workgroup leaves to the accurate form (state 2): bit k for its
  // k-th row (k < 64), else the kL1Redo marker in l1 (rows past 64 x grid)
  uint64_t redo = 0;
  bool redo_far = false;
  int it = 0;
  for (; row < rows; row += gridDim.x, ++it) {
    const int b = it & 1;
    const __amdgpu_buffer_rsrc_t rt = rsrc(tgt, ld_t, row);
    uint4 tb[RES_U];
#pragma unroll
    for (int u = 0; u < RES_U; ++u) tb[u] = res_load(rt, voff, u);
    // this thread's tail element, if any; kept raw until the end of pass 1, so
    // the wait for it does not also wait for every load issued before it
    uint16_t ta_raw = 0, da_raw = 0;
    if (tid < ntail) {
      ta_raw = tgt[row * ld_t + nvec * 8 + tid];
      da_raw = dft[row * ld_d + nvec * 8 + tid];
    }

    // ---- pass 1: sums of both rows against lazily moved references; target
    // chunks j < RES_JL kept in LDS ----
    float cx = kNegInf, sx = 0.0f, cy = kNegInf, sy = 0.0f;
#pragma unroll
    for (int j = 0; j < RES_JD; ++j) {
      const uint4 w = tb[j % RES_U];
      if (j + RES_U < RES_JD) tb[j % RES_U] = res_load(rt, voff, j + RES_U);
      if (j < nj) {
        float v[8];
        unpack8(w, v);
        lazy_add<8>(cx, sx, v);
        if (j < RES_JL) keep[j][tid] = w;
        unpack8(d[j], v);
        lazy_add<8>(cy, sy, v);
      }
    }
    uint32_t tr = ta_raw, dr = da_raw;
    asm volatile("" : "+v"(tr), "+v"(dr));  // keeps the conversion (and its wait) here
    const float ta = __uint_as_float(tr << 16), da = __uint_as_float(dr << 16);
    if (tid < ntail) {
      lazy_add<1>(cx, sx, &ta);
      lazy_add<1>(cy, sy, &da);
    }
    // the first re-read target chunks go out before the merge
#pragma unroll
    for (int u = 0; u < RES_U; ++u)
      if (RES_JL + u < RES_JD) tb[u] = res_load(rt, voff, RES_JL + u);

    // merge: wave maximum of the references, rescaled wave sums (lane 0),
    // then every wave combines the NW wave states itself in a fixed order
    {
      const float Mx = wave_max_all(cx), My = wave_max_all(cy);
      const float wx = wave_sum_all(sx * ref_scale(cx, Mx));
      const float wy = wave_sum_all(sy * ref_scale(cy, My));
      if (lane == 0) {
        red_a[b][wave][0] = Mx;
        red_a[b][wave][1] = wx;
        red_a[b][wave][2] = My;
        red_a[b][wave][3] = wy;
      }
    }
    __syncthreads();
    if (tid == 0 && it > 0) finish(row - gridDim.x, b ^ 1, prev_state);
    float Mx = red_a[b][0][0], My = red_a[b][0][2];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      Mx = fmaxf(Mx, red_a[b][w][0]);
      My = fmaxf(My, red_a[b][w][2]);
    }
    float Sx = 0.0f, Sy = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      Sx += red_a[b][w][1] * ref_scale(red_a[b][w][0], Mx);
      Sy += red_a[b][w][3] * ref_scale(red_a[b][w][2], My);
    }
    const Norm nx = make_norm(Mx, Sx), ny = make_norm(My, Sy);  // base-2 normalisers of each row
    const bool ok = norm_ok(nx) && norm_ok(ny);

    // ---- pass 2: sum |p - q|; the next row's draft chunks replace the used ones ----
    // (a row with a non-finite normaliser runs it too, to keep the next row's
    // loads going; its sum is discarded)
    const __amdgpu_buffer_rsrc_t rn = rsrc(dft, ld_d, row + gridDim.x);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < RES_JD; ++j) {
      uint4 w;
      if (j < RES_JL) {
        w = keep[j][tid];
      } else {
        w = tb[(j - RES_JL) % RES_U];
        if (j + RES_U < RES_JD) tb[(j - RES_JL) % RES_U] = res_load(rt, voff, j + RES_U);
      }
      if (j < nj) {
        float a[8], c[8];
        unpack8(w, a);
        unpack8(d[j], c);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += absdiff<false>(a[i], c[i], nx, ny, kLog2eBf16);
      }
      d[j] = res_load(rn, voff, j);
    }
    if (tid < ntail) acc += absdiff<false>(ta, da, nx, ny, kLog2eBf16);
    acc = wave_sum_all(acc);
    if (lane == 0) red_b[b][wave] = acc;  // summed after the next row's barrier
    prev_state = !ok ? 0 : (fabsf(nx.m) < kBigRef && fabsf(ny.m) < kBigRef) ? 1 : 2;
    if (prev_state == 2) {
      if (it < 64)
        redo |= uint64_t(1) << it;
      else
        redo_far = true;
    }
  }
  __syncthreads();
  if (tid == 0 && it > 0) finish(row - gridDim.x, (it - 1) & 1, prev_state);
  if (redo == 0 && !redo_far) return;  // (the same for every thread of the workgroup)
  // rows whose maxima passed 2^13: done again here by the two-pass form,
  // which takes the accurate exponent form on them
  __syncthreads();  // thread 0's markers are visible to the whole workgroup
  int k = 0;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x, ++k) {
    const bool mine = k < 64 ? ((redo >> k) & 1) != 0 : l1[r] == kL1Redo;
    if (!mine) continue;
    l1_row<VS_BF16, RES_NT, 4>(tgt, ld_t, dft, ld_d, V, r, l1, accept);
    __syncthreads();  // this row's last LDS reads come before the next row's writes
  }
}

// 256 threads x 8 loads in flight: several rows per CU overlap their passes
// (measured at T=2048, V=151,936: 359 us against 410 us for one
// 1024-thread row per CU with plain loads)
constexpr int kL1Threads = 256;
constexpr int kL1Unroll = 8;

// ---------------------------------------------------------------------------
// The weighted L1 distillation loss and its draft-logit gradient (DeepSpec PR
// #87, Purpose and Test Plan: the distance is computed once and feeds both
// accept_rate and the weighted L1 loss num / den, num = sum_t w_t L1_t,
// den = sum_t w_t; the loss's gradient goes to the draft logits):
//   d L1_t / d b_v = q_v (s_v - S_t),  s_v = sign(q_v - p_v),  S_t = sum_u s_u q_u.
// Every row is split over S workgroups (slices; S = 2 .. 8, more when the
// batch has few rows per CU, so that small batches still fill the chip).
// l1_part1_kernel, l1_part2_kernel: the L1 kernel's two passes, the second
//   also summing S_t, each into per-slice partials.
// l1_loss_kernel: one 1024-thread workgroup: adds each row's partials in slice order
//   (l1, accept, S_t), then num and den in a fixed order.
// l1_grad_kernel: one pass over each slice: recomputes p_v, q_v and their
//   sign with the same instructions as the stats pass, and writes
//   grad_scale (w_t / den) q_v (s_v - S_t).
// A row of weight 0 adds nothing to num and gets a zero gradient (a loss
// mask), even if its distance is NaN.
// ---------------------------------------------------------------------------
constexpr int kLossThreads = 256;
constexpr int kLossUnroll = 8;

struct RowStats {
  float mx, l2sx, my, l2sy, S;  // normalisers of both rows (base 2), sum s q; mx = NaN on a bad row
};

template <bool ACC>
__device__ __forceinline__ void pq_pair(float a, float b, const Norm& x, const Norm& y, float l2e, float& p, float& q) {
  if (ACC) {
    p = exp2_hw(__builtin_fmaf(a, l2e, -x.m) - x.l2s);
    q = exp2_hw(__builtin_fmaf(b, l2e, -y.m) - y.l2s);
  } else {
    p = exp2_hw(__builtin_fmaf(a, l2e, -x.l));
    q = exp2_hw(__builtin_fmaf(b, l2e, -y.l));
  }
}
__device__ __forceinline__ float sgn(float d) { return d > 0.0f ? 1.0f : d < 0.0f ? -1.0f : 0.0f; }

// Calls f(a, b, n) on this thread's share of a row pair: U 16-byte chunks per
// step in flight (n = VEC values each), then the remaining chunks, then the
// scalar tail (n = 1).
// (A row split over several workgroups runs this as thread g of G per row:
// g = slice * NT + threadIdx.x, G = slices * NT.)
template <int DT, int NT, int U, class F>
__device__ __forceinline__ void row_pairs(const char* trow, const char* drow, int64_t nvec, int64_t V, F f,
                                          int g = int(threadIdx.x), int64_t G = NT) {
  constexpr int VEC = DT == VS_BF16 ? 8 : 4;
  int64_t q = g;
  for (; q + int64_t(U - 1) * G < nvec; q += int64_t(U) * G) {
    float a[U][VEC], b[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load_chunk<DT>(trow, q + u * G, a[u]);
      load_chunk<DT>(drow, q + u * G, b[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) f(a[u], b[u], VEC);
  }
  for (; q < nvec; q += G) {
    float a[VEC], b[VEC];
    load_chunk<DT>(trow, q, a);
    load_chunk<DT>(drow, q, b);
    f(a, b, VEC);
  }
  for (int64_t i = nvec * VEC + g; i < V; i += G) {
    float a = load_one<DT>(trow, i), b = load_one<DT>(drow, i);
    f(&a, &b, 1);
  }
}

// The stats passes with each row split over S workgroups (slices).  Slice s
// of row t is thread g = s * NT + threadIdx.x of S * NT.  l1_part1_kernel: each slice's online maxima and sums of both
// rows (merged in its workgroup as in the one-workgroup form) into
// part1[t * S + s].  l1_part2_kernel: every slice merges the row's S partials
// in slice order (all get the same normalisers), runs pass 2 over its share
// and writes its sums of |p - q| and sign(q - p) q into part2[t * S + s];
// slice 0 writes the row's normalisers.  l1_loss_kernel then adds each row's
// S partial sums in slice order.
template <int NT>
__device__ __forceinline__ void block_pair(Part& px, Part& py, float (*red)[4], float* fin) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  px = wave_merge_to_lane0(px);
  py = wave_merge_to_lane0(py);
  if ((tid & 63) == 0) {
    red[tid >> 6][0] = px.m;
    red[tid >> 6][1] = px.s;
    red[tid >> 6][2] = py.m;
    red[tid >> 6][3] = py.s;
  }
  __syncthreads();
  if (tid < 64) {
    Part qx{kNegInf, 0.0f, 0.0f}, qy{kNegInf, 0.0f, 0.0f};
    if (tid < NW) {
      qx = Part{red[tid][0], red[tid][1], 0.0f};
      qy = Part{red[tid][2], red[tid][3], 0.0f};
    }
    qx = wave_merge_to_lane0(qx);
    qy = wave_merge_to_lane0(qy);
    if (tid == 0) {
      fin[0] = qx.m;
      fin[1] = qx.s;
      fin[2] = qy.m;
      fin[3] = qy.s;
    }
  }
  __syncthreads();
}

template <int DT, int NT, int U>
__global__ __launch_bounds__(NT) void l1_part1_kernel(const void* __restrict__ tgt, int64_t ld_t,
                                                      const void* __restrict__ dft, int64_t ld_d, int64_t V, int S,
                                                      float4* __restrict__ part1) {
  constexpr int VEC = DT == VS_BF16 ? 8 : 4;
  constexpr int ES = DT == VS_BF16 ? 2 : 4;
  constexpr int NW = NT / 64;
  constexpr float l2e = DT == VS_BF16 ? kLog2eBf16 : kLog2e;
  __shared__ float red[NW][4];
  __shared__ float fin[4];
  const int64_t row = blockIdx.x / S;
  const int sl = int(blockIdx.x - row * S);
  const char* trow = static_cast<const char*>(tgt) + row * ld_t * ES;
  const char* drow = static_cast<const char*>(dft) + row * ld_d * ES;
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(trow) | reinterpret_cast<uintptr_t>(drow)) & 15) == 0;
  const int64_t nvec = vec_ok ? V / VEC : 0;
  float mx = kNegInf, sx = 0.0f, my = kNegInf, sy = 0.0f;
  row_pairs<DT, NT, U>(
      trow, drow, nvec, V,
      [&](const float* a, const float* b, int n) {
        online(mx, sx, a, n, l2e);
        online(my, sy, b, n, l2e);
      },
      sl * NT + int(threadIdx.x), int64_t(S) * NT);
  Part px{mx * l2e, sx, 0.0f}, py{my * l2e, sy, 0.0f};
  block_pair<NT>(px, py, red, fin);
  if (threadIdx.x == 0) part1[blockIdx.x] = make_float4(fin[0], fin[1], fin[2], fin[3]);
}

template <int DT, int NT, int U>
__global__ __launch_bounds__(NT) void l1_part2_kernel(const void* __restrict__ tgt, int64_t ld_t,
                                                      const void* __restrict__ dft, int64_t ld_d, int64_t V, int S,
                                                      const float4* __restrict__ part1, float2* __restrict__ part2,
                                                      RowStats* __restrict__ stats) {
  constexpr int VEC = DT == VS_BF16 ? 8 : 4;
  constexpr int ES = DT == VS_BF16 ? 2 : 4;
  constexpr int NW = NT / 64;
  constexpr float l2e = DT == VS_BF16 ? kLog2eBf16 : kLog2e;
  __shared__ float red[NW][2];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x / S;
  const int sl = int(blockIdx.x - row * S);
  Part qx{kNegInf, 0.0f, 0.0f}, qy{kNegInf, 0.0f, 0.0f};
  for (int k = 0; k < S; ++k) {
    const float4 p = part1[row * S + k];
    qx = merge(qx, Part{p.x, p.y, 0.0f});
    qy = merge(qy, Part{p.z, p.w, 0.0f});
  }
  const Norm nx = make_norm(qx.m, qx.s), ny = make_norm(qy.m, qy.s);
  if (!(norm_ok(nx) && norm_ok(ny))) {
    if (tid == 0) {
      const float nan = __builtin_nanf("");
      part2[blockIdx.x] = make_float2(nan, nan);
      if (sl == 0) stats[row] = RowStats{nan, nan, nan, nan, nan};
    }
    return;
  }
  const char* trow = static_cast<const char*>(tgt) + row * ld_t * ES;
  const char* drow = static_cast<const char*>(dft) + row * ld_d * ES;
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(trow) | reinterpret_cast<uintptr_t>(drow)) & 15) == 0;
  const int64_t nvec = vec_ok ? V / VEC : 0;
  float d1 = 0.0f, ds = 0.0f;
  auto pass2 = [&](auto acc_form) {
    constexpr bool ACC = decltype(acc_form)::value;
    row_pairs<DT, NT, U>(
        trow, drow, nvec, V,
        [&](const float* a, const float* b, int n) {
          for (int i = 0; i < n; ++i) {
            float pp, qq;
            pq_pair<ACC>(a[i], b[i], nx, ny, l2e, pp, qq);
            d1 += fabsf(pp - qq);
            ds = __builtin_fmaf(sgn(qq - pp), qq, ds);
          }
        },
        sl * NT + tid, int64_t(S) * NT);
  };
  if (norms_big(nx, ny))
    pass2(std::true_type{});
  else
    pass2(std::false_type{});
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o1 = shfl_down_f(d1, off), o2 = shfl_down_f(ds, off);
    if ((tid & ((off << 1) - 1)) == 0) {
      d1 += o1;
      ds += o2;
    }
  }
  if ((tid & 63) == 0) {
    red[tid >> 6][0] = d1;
    red[tid >> 6][1] = ds;
  }
  __syncthreads();
  if (tid == 0) {
    float v = 0.0f, Sv = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      v += red[w][0];
      Sv += red[w][1];
    }
    part2[blockIdx.x] = make_float2(v, Sv);
    if (sl == 0) stats[row] = RowStats{nx.m, nx.l2s, ny.m, ny.l2s, 0.0f};
  }
}

// num = sum_t w_t l1_t over rows of nonzero weight, den = sum_t w_t: thread i
// takes rows i, i + 256, ... in order, then a fixed tree.  out = {num, den, num / den}.
// Row t's distance and sum s q are first added up from its S partials in
// slice order, and l1, accept and the row's S_t written.
constexpr int kLossFinThreads = 1024;
__global__ __launch_bounds__(kLossFinThreads) void l1_loss_kernel(float* __restrict__ l1, float* __restrict__ accept,
                                                               const float* __restrict__ weights, int64_t rows,
                                                               float* __restrict__ out, const float2* __restrict__ part2,
                                                               int S, RowStats* __restrict__ stats) {
  __shared__ float sn[kLossFinThreads], sd[kLossFinThreads];
  const int tid = threadIdx.x;
  float n = 0.0f, d = 0.0f;
  for (int64_t t = tid; t < rows; t += kLossFinThreads) {
    const bool ok = stats[t].mx == stats[t].mx;
    float v = 0.0f, Sv = 0.0f;
    for (int k = 0; k < S; ++k) {
      const float2 p = part2[t * S + k];
      v += p.x;
      Sv += p.y;
    }
    const float nan = __builtin_nanf("");
    const float lt = ok ? fminf(fmaxf(v, 0.0f), 2.0f) : nan;
    l1[t] = lt;
    if (accept) accept[t] = ok ? fminf(fmaxf(1.0f - 0.5f * lt, 0.0f), 1.0f) : nan;
    if (ok) stats[t].S = Sv;
    const float w = weights ? weights[t] : 1.0f;
    if (w != 0.0f) n = __builtin_fmaf(w, lt, n);
    d += w;
  }
  sn[tid] = n;
  sd[tid] = d;
  __syncthreads();
  for (int h = kLossFinThreads / 2; h > 0; h >>= 1) {
    if (tid < h) {
      sn[tid] += sn[tid + h];
      sd[tid] += sd[tid + h];
    }
    __syncthreads();
  }
  if (tid == 0) {
    out[0] = sn[0];
    out[1] = sd[0];
    out[2] = sn[0] / sd[0];
  }
}

__device__ __forceinline__ uint32_t bf16_rne(float v) {
  // round to nearest even (NaN kept quiet)
  const uint32_t u = __float_as_uint(v);
  return (v != v) ? ((u >> 16) | 0x40u) : ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Two fp32 values as packed bf16, a in the low half: the hardware's round to
// nearest even (v_cvt_pk_bf16_f32), the same result as bf16_rne off NaN.
typedef __bf16 l1_bf16x2 __attribute__((ext_vector_type(2)));
typedef float l1_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16_hw(float a, float b) {
  const l1_f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, l1_bf16x2));
}

template <int GDT>
__device__ __forceinline__ void store_one(void* g, int64_t i, float v) {
  if (GDT == VS_BF16)
    static_cast<uint16_t*>(g)[i] = uint16_t(bf16_rne(v));
  else
    static_cast<float*>(g)[i] = v;
}

// n gradient values of consecutive elements starting at element i (16-byte
// aligned when n > 1)
template <int GDT>
__device__ __forceinline__ void store_run(void* g, int64_t i, const float* v, int n) {
  if (n == 8 && GDT == VS_BF16) {
    uint4 w;
    w.x = pack_bf16_hw(v[0], v[1]);
    w.y = pack_bf16_hw(v[2], v[3]);
    w.z = pack_bf16_hw(v[4], v[5]);
    w.w = pack_bf16_hw(v[6], v[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(g) + i) = w;
  } else if (n % 4 == 0 && GDT == VS_F32) {
    for (int k = 0; k < n; k += 4)
      *reinterpret_cast<float4*>(static_cast<float*>(g) + i + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
  } else {
    for (int k = 0; k < n; ++k) store_one<GDT>(g, i + k, v[k]);
  }
}

template <int DT, int GDT, int NT>
__global__ __launch_bounds__(NT) void l1_grad_kernel(const void* __restrict__ tgt, int64_t ld_t,
                                                     const void* __restrict__ dft, int64_t ld_d, int64_t V,
                                                     const float* __restrict__ weights, float grad_scale,
                                                     const RowStats* __restrict__ stats,
                                                     const float* __restrict__ loss_out, void* __restrict__ grad,
                                                     int64_t ld_g, int S) {
  constexpr int VEC = DT == VS_BF16 ? 8 : 4;
  constexpr int ES = DT == VS_BF16 ? 2 : 4;
  constexpr int GS = GDT == VS_BF16 ? 2 : 4;
  constexpr float l2e = DT == VS_BF16 ? kLog2eBf16 : kLog2e;
  // row t over S workgroups: this is thread g of the row's G (each gradient
  // element is computed on its own, so the split changes no value)
  const int64_t row = blockIdx.x / S;
  const int tid = int(blockIdx.x - row * S) * NT + int(threadIdx.x);
  const int64_t G = int64_t(S) * NT;
  const float w = weights ? weights[row] : 1.0f;
  const RowStats st = stats[row];
  const char* trow = static_cast<const char*>(tgt) + row * ld_t * ES;
  const char* drow = static_cast<const char*>(dft) + row * ld_d * ES;
  const int64_t g0 = row * ld_g;
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(trow) | reinterpret_cast<uintptr_t>(drow) |
                        (reinterpret_cast<uintptr_t>(grad) + uintptr_t(g0) * GS)) & 15) == 0;
  const int64_t nvec = vec_ok ? V / VEC : 0;
  if (w == 0.0f || !(st.mx == st.mx)) {  // masked row: zeros; a bad row: NaN
    const float v = w == 0.0f ? 0.0f : __builtin_nanf("");
    for (int64_t i = tid; i < V; i += G) store_one<GDT>(grad, g0 + i, v);
    return;
  }
  const float scale = grad_scale * (w / loss_out[1]);
  const Norm nx{st.mx, st.l2sx, st.mx + st.l2sx}, ny{st.my, st.l2sy, st.my + st.l2sy};
  auto run = [&](auto acc_form) {
    constexpr bool ACC = decltype(acc_form)::value;
    auto grads = [&](const float* a, const float* b, int n, float* g) {
      for (int i = 0; i < n; ++i) {
        float pp, qq;
        pq_pair<ACC>(a[i], b[i], nx, ny, l2e, pp, qq);
        g[i] = scale * (qq * (sgn(qq - pp) - st.S));
      }
    };
    int64_t q = tid;
    constexpr int U = 4;
    for (; q + int64_t(U - 1) * G < nvec; q += int64_t(U) * G) {
      float a[U][VEC], b[U][VEC];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        load_chunk<DT>(trow, q + u * G, a[u]);
        load_chunk<DT>(drow, q + u * G, b[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float g[VEC];
        grads(a[u], b[u], VEC, g);
        store_run<GDT>(grad, g0 + (q + u * G) * VEC, g, VEC);
      }
    }
    for (; q < nvec; q += G) {
      float a[VEC], b[VEC], g[VEC];
      load_chunk<DT>(trow, q, a);
      load_chunk<DT>(drow, q, b);
      grads(a, b, VEC, g);
      store_run<GDT>(grad, g0 + q * VEC, g, VEC);
    }
    for (int64_t i = nvec * VEC + tid; i < V; i += G) {
      const float a = load_one<DT>(trow, i), b = load_one<DT>(drow, i);
      float g;
      grads(&a, &b, 1, &g);
      store_one<GDT>(grad, g0 + i, g);
    }
  };
  if (norms_big(nx, ny))
    run(std::true_type{});
  else
    run(std::false_type{});
}

}  // namespace

size_t l1_workspace_bytes(int64_t rows, int64_t V) {
  (void)rows;
  (void)V;
  return 0;
}

int launch_l1(LogitsArg target, LogitsArg draft, int64_t rows, int64_t V, float* l1, float* accept, void* workspace,
              void* stream) {
  (void)workspace;
  if (rows <= 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool aligned = ((reinterpret_cast<uintptr_t>(target.ptr) | reinterpret_cast<uintptr_t>(draft.ptr)) & 15) == 0 &&
                       (target.ld & 7) == 0 && (draft.ld & 7) == 0;
  if (target.dtype == VS_BF16 && aligned && V >= kResMinV && V <= kResMaxVec * 8 + 7) {
    int ncu = 0;
    if (const int e = device_cu_count(&ncu)) return e;
    const int64_t grid = rows < ncu ? rows : ncu;
    l1_resident_kernel<<<dim3(unsigned(grid)), dim3(RES_NT), 0, s>>>(
        static_cast<const uint16_t*>(target.ptr), target.ld, static_cast<const uint16_t*>(draft.ptr), draft.ld, rows, V,
        l1, accept);
    return int(hipGetLastError());
  }
  if (target.dtype == VS_BF16) {
    l1_kernel<VS_BF16, kL1Threads, kL1Unroll><<<dim3(unsigned(rows)), dim3(kL1Threads), 0, s>>>(
        target.ptr, target.ld, draft.ptr, draft.ld, V, l1, accept);
  } else {
    l1_kernel<VS_F32, kL1Threads, kL1Unroll><<<dim3(unsigned(rows)), dim3(kL1Threads), 0, s>>>(
        target.ptr, target.ld, draft.ptr, draft.ld, V, l1, accept);
  }
  return int(hipGetLastError());
}

// Slices per row: enough for about 4 workgroups per CU, at least 2 (measured
// faster than one workgroup per row even on large batches) and at most 8.
constexpr int kLossMaxSlices = 8;

int loss_slices(int64_t rows, int ncu) {
  const int64_t s = (4 * int64_t(ncu) + rows - 1) / rows;
  return int(s < 2 ? 2 : s > kLossMaxSlices ? kLossMaxSlices : s);
}

size_t l1_loss_workspace_bytes(int64_t rows) {
  return size_t(rows) * sizeof(RowStats) + 256 + 16 + size_t(rows) * kLossMaxSlices * (sizeof(float4) + sizeof(float2));
}

int launch_l1_loss(LogitsArg target, LogitsArg draft, int64_t rows, int64_t V, const float* weights,
                   float grad_scale, float* l1, float* accept, float* loss_out, void* grad, int grad_dtype,
                   int64_t ld_grad, void* workspace, void* stream) {
  if (rows <= 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int ncu = 0;
  if (const int e = device_cu_count(&ncu)) return e;
  const int S = loss_slices(rows, ncu);
  RowStats* stats = static_cast<RowStats*>(workspace);
  // partials after the stats and the 256 + 16 bytes kept for alignment (16-byte aligned)
  const uintptr_t pbase = (reinterpret_cast<uintptr_t>(stats + rows) + 255) & ~uintptr_t(255);
  float4* part1 = reinterpret_cast<float4*>(pbase);
  float2* part2 = reinterpret_cast<float2*>(part1 + rows * S);
  const dim3 g{unsigned(rows * S)}, b{unsigned(kLossThreads)};
  if (target.dtype == VS_BF16) {
    l1_part1_kernel<VS_BF16, kLossThreads, kLossUnroll><<<g, b, 0, s>>>(target.ptr, target.ld, draft.ptr, draft.ld, V,
                                                                        S, part1);
    l1_part2_kernel<VS_BF16, kLossThreads, kLossUnroll><<<g, b, 0, s>>>(target.ptr, target.ld, draft.ptr, draft.ld, V,
                                                                        S, part1, part2, stats);
  } else {
    l1_part1_kernel<VS_F32, kLossThreads, kLossUnroll><<<g, b, 0, s>>>(target.ptr, target.ld, draft.ptr, draft.ld, V,
                                                                       S, part1);
    l1_part2_kernel<VS_F32, kLossThreads, kLossUnroll><<<g, b, 0, s>>>(target.ptr, target.ld, draft.ptr, draft.ld, V,
                                                                       S, part1, part2, stats);
  }
  l1_loss_kernel<<<dim3(1), dim3(kLossFinThreads), 0, s>>>(l1, accept, weights, rows, loss_out, part2, S, stats);
  if (grad) {
    if (target.dtype == VS_BF16 && grad_dtype == VS_BF16)
      l1_grad_kernel<VS_BF16, VS_BF16, kLossThreads><<<g, b, 0, s>>>(target.ptr, target.ld, draft.ptr, draft.ld, V,
                                                                     weights, grad_scale, stats, loss_out, grad,
                                                                     ld_grad, S);
    else if (target.dtype == VS_BF16)
      l1_grad_kernel<VS_BF16, VS_F32, kLossThreads><<<g, b, 0, s>>>(target.ptr, target.ld, draft.ptr, draft.ld, V,
                                                                    weights, grad_scale, stats, loss_out, grad,
                                                                    ld_grad, S);
    else if (grad_dtype == VS_BF16)
      l1_grad_kernel<VS_F32, VS_BF16, kLossThreads><<<g, b, 0, s>>>(target.ptr, target.ld, draft.ptr, draft.ld, V,
                                                                    weights, grad_scale, stats, loss_out, grad,
                                                                    ld_grad, S);
    else
      l1_grad_kernel<VS_F32, VS_F32, kLossThreads><<<g, b, 0, s>>>(target.ptr, target.ld, draft.ptr, draft.ld, V,
                                                                   weights, grad_scale, stats, loss_out, grad,
                                                                   ld_grad, S);
  }
  return int(hipGetLastError());
}

}  // namespace vs
