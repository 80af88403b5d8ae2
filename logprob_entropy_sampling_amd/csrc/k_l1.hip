// Draft/target softmax L1 distance (DeepSpec PR #87, Purpose: the per-token
// distance sum_v |P_v - Q_v| computed once and shared by
// accept_rate = clamp(1 - 0.5 * L1, 0, 1) and the L1 loss).
//
// One workgroup per token row.  Pass 1 streams both rows once and folds each
// into an online (max, sum-exp) state; pass 2 streams them again and sums
// |2^(u - M - log2 S) - 2^(w - M' - log2 S')|, the normalisers folded into the
// exponent so each probability is one FMA + one v_exp_f32.  No probability
// vector is stored anywhere.  Identical rows give exactly 0: both sides run
// the same instructions on the same bits.
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
