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
__device__ __forceinline__ void online(float& m, float& s, const float* v, int n) {
  float bm = v[0];
  for (int i = 1; i < n; ++i) bm = fmaxf(bm, v[i]);
  const float nm = fmaxf(m, bm);
  if (nm == kNegInf) {  // only -inf so far, or a NaN that fmaxf dropped
    for (int i = 0; i < n; ++i)
      if (v[i] != v[i]) s = __builtin_nanf("");
    return;
  }
  const float c = nm * kLog2e;
  s *= exp2_hw(m * kLog2e - c);  // exactly 1 when the max did not move; 0 from -inf
  for (int i = 0; i < n; ++i) s += exp2_hw(__builtin_fmaf(v[i], kLog2e, -c));
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

// |p - q| of one element pair, the normalisers folded into the exponents
__device__ __forceinline__ float absdiff(float a, float b, float lx, float ly) {
  return fabsf(exp2_hw(__builtin_fmaf(a, kLog2e, -lx)) - exp2_hw(__builtin_fmaf(b, kLog2e, -ly)));
}

// NT threads per row; U vector chunks per thread in flight per pass step.
template <int DT, int NT, int U>
__global__ __launch_bounds__(NT) void l1_kernel(const void* __restrict__ tgt, int64_t ld_t, const void* __restrict__ dft,
                                                int64_t ld_d, int64_t V, float* __restrict__ l1,
                                                float* __restrict__ accept) {
  constexpr int VEC = DT == VS_BF16 ? 8 : 4;
  constexpr int ES = DT == VS_BF16 ? 2 : 4;
  constexpr int NW = NT / 64;
  __shared__ float red[NW][4];
  const int64_t row = blockIdx.x;
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
      online(mx, sx, a[u], VEC);
      online(my, sy, b[u], VEC);
    }
  }
  for (; q < nvec; q += NT) {
    float a[VEC], b[VEC];
    load_chunk<DT>(trow, q, a);
    load_chunk<DT>(drow, q, b);
    online(mx, sx, a, VEC);
    online(my, sy, b, VEC);
  }
  for (int64_t i = tail0 + tid; i < V; i += NT) {
    float a = load_one<DT>(trow, i), b = load_one<DT>(drow, i);
    online(mx, sx, &a, 1);
    online(my, sy, &b, 1);
  }
  // block merge (fixed tree): wave tree, then wave 0 over the NW wave states;
  // the merge works in base-2 units
  Part px = wave_merge_to_lane0(Part{mx * kLog2e, sx, 0.0f});
  Part py = wave_merge_to_lane0(Part{my * kLog2e, sy, 0.0f});
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
      fin[0] = qx.m + log2_hw(qx.s);  // base-2 LSE of the target row
      fin[1] = qy.m + log2_hw(qy.s);
    }
  }
  __syncthreads();
  const float lx = fin[0], ly = fin[1];
  const bool ok = lx > -__builtin_inff() && lx < __builtin_inff() && ly > -__builtin_inff() && ly < __builtin_inff();
  if (!ok) {
    if (tid == 0) {
      l1[row] = __builtin_nanf("");
      if (accept) accept[row] = __builtin_nanf("");
    }
    return;
  }

  // ---- pass 2: sum |p - q| ----
  float acc = 0.0f;
  q = tid;
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
      for (int i = 0; i < VEC; ++i) acc += absdiff(a[u][i], b[u][i], lx, ly);
  }
  for (; q < nvec; q += NT) {
    float a[VEC], b[VEC];
    load_chunk<DT>(trow, q, a);
    load_chunk<DT>(drow, q, b);
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc += absdiff(a[i], b[i], lx, ly);
  }
  for (int64_t i = tail0 + tid; i < V; i += NT) {
    const float a = load_one<DT>(trow, i), b = load_one<DT>(drow, i);
    acc += absdiff(a, b, lx, ly);
  }
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
  for (int i = 0; i < N; ++i) cs += exp2_hw(__builtin_fmaf(v[i], kLog2e, -c));
  if (!(cs < 0x1p64f)) {
    float bm = v[0];
#pragma unroll
    for (int i = 1; i < N; ++i) bm = fmaxf(bm, v[i]);
    const float nc = fmaxf(c, bm * kLog2e);
    cs = 0.0f;
    if (nc == kNegInf) {  // only -inf so far (or NaNs that fmaxf dropped)
#pragma unroll
      for (int i = 0; i < N; ++i)
        if (v[i] != v[i]) cs = __builtin_nanf("");
    } else {
      s *= exp2_hw(c - nc);  // 0 from the initial -inf
      c = nc;
#pragma unroll
      for (int i = 0; i < N; ++i) cs += exp2_hw(__builtin_fmaf(v[i], kLog2e, -c));
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
  // row r's L1 from the pass-2 partials of buffer b (thread 0)
  auto finish = [&](int64_t r, int b, bool ok) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red_b[b][w];
    const float dd = ok ? fminf(fmaxf(v, 0.0f), 2.0f) : __builtin_nanf("");
    l1[r] = dd;
    if (accept) accept[r] = ok ? fminf(fmaxf(1.0f - 0.5f * dd, 0.0f), 1.0f) : __builtin_nanf("");
  };

  int64_t row = blockIdx.x;
  uint4 d[RES_JD];
  {
    const __amdgpu_buffer_rsrc_t rd = rsrc(dft, ld_d, row);
#pragma unroll
    for (int j = 0; j < RES_JD; ++j) d[j] = res_load(rd, voff, j);
  }
  bool prev_ok = false;
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
    if (tid == 0 && it > 0) finish(row - gridDim.x, b ^ 1, prev_ok);
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
    const float lx = Mx + log2_hw(Sx);  // base-2 log-sum-exp of each row
    const float ly = My + log2_hw(Sy);
    const bool ok = lx > -__builtin_inff() && lx < __builtin_inff() && ly > -__builtin_inff() && ly < __builtin_inff();

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
        for (int i = 0; i < 8; ++i) acc += absdiff(a[i], c[i], lx, ly);
      }
      d[j] = res_load(rn, voff, j);
    }
    if (tid < ntail) acc += absdiff(ta, da, lx, ly);
    acc = wave_sum_all(acc);
    if (lane == 0) red_b[b][wave] = acc;  // summed after the next row's barrier
    prev_ok = ok;
  }
  __syncthreads();
  if (tid == 0 && it > 0) finish(row - gridDim.x, (it - 1) & 1, prev_ok);
}

// 256 threads x 8 loads in flight: several rows per CU overlap their passes
// (measured at T=2048, V=151,936: 359 us against 410 us for one
// 1024-thread row per CU with plain loads)
constexpr int kL1Threads = 256;
constexpr int kL1Unroll = 8;

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
    // CU count of the current device, cached per device (a benign race: every
    // writer stores the same value)
    static int cu_count[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return int(hipErrorInvalidDevice);
    int ncu = dev < 64 ? cu_count[dev] : 0;
    if (ncu <= 0) {
      if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
        return int(hipErrorInvalidDevice);
      if (dev < 64) cu_count[dev] = ncu;
    }
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

}  // namespace vs
