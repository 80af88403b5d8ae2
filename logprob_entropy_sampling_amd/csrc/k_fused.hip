// Fused LM-head sweep: bf16 MFMA projection hidden x W^T with the softmax
// statistics folded into the epilogue, so no logit is ever written to memory.
//
// The op is the "chunked projection -> fixed-order LSE -> selected logprob"
// of xorl issue #71 section 1; the full-vocabulary entropy path of SkyRL PR
// #2004.  Design for gfx950 (not the pages' PyTorch chunk loop):
//   * output tile = 256 vocabulary rows x 256 token columns per workgroup,
//     4 waves of 128 x 128, v_mfma_f32_32x32x16_bf16 with fp32 accumulators;
//   * the MFMA's A operand is the weight (vocabulary on the M axis), B the
//     hidden state (tokens on the N axis), so every lane holds one token
//     column and 64 vocabulary rows: the max / sum-exp / sum p*z fold is
//     lane-local, with one cross-half and one cross-wave merge per tile;
//   * K is swept in 32-wide slices staged through double-buffered LDS with
//     a 16-byte-chunk XOR swizzle (conflict-free fragment reads);
//   * workgroup ids are remapped so each XCD walks a contiguous range of
//     vocabulary tiles, all token tiles of one vocabulary tile back to back:
//     a weight tile is fetched from HBM once and reused from that XCD's L2.
#include "common.h"
#include "launch.h"

namespace vs {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BV = kFusedTileV;  // 256 vocabulary rows
constexpr int BT = kFusedTileT;  // 256 token rows
constexpr int BK = 32;           // K slice per stage
constexpr int CH = BK / 8;       // 16-byte chunks per row per stage (4)
constexpr int NT = 256;          // threads (4 waves: 2 along V x 2 along T)
constexpr int LOADS = BV * CH / NT;  // 16-byte loads per thread per operand per stage (4)

__device__ __forceinline__ int swz(int r, int c) { return r * CH + (c ^ ((r >> 1) & 3)); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }


// ---- epilogue: per token column, fold this tile's 256 vocabulary rows ----
// acc[i][j][r] holds vocabulary row  wv*128 + 32i + 8(r/4) + 4*lh + (r%4)
// and token column                   wt*128 + 32j + lr          (lr = lane & 31, lh = lane >> 5).
// Each lane folds its 64 rows of one column into (max, sum 2^(u-max), sum 2^(u-max)(u-max));
// the two half-waves and the two V-direction waves are merged, and one partial per
// (token, vocabulary tile) is written.  The lane holding the target id stores its raw logit.
// `red` is >= 3 KiB of LDS that no wave reads any more.
__device__ __forceinline__ void tile_epilogue(f32x16 (&acc)[4][4], float* red, int64_t v0, int64_t t0, int vt,
                                              int64_t rows_valid, int64_t V, const float* __restrict__ temp,
                                              float temp_scalar, const int64_t* __restrict__ targets,
                                              const int32_t* __restrict__ row_map, int n_vtiles,
                                              float4* __restrict__ partials, float* __restrict__ zy_raw) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wv = w & 1;
  const int wt = w >> 1;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  // vocabulary rows of this wave that exist (the last tile may be ragged)
  const int vlim = int(V - v0 < BV ? V - v0 : BV) - wv * 128;  // rows r of the wave with r < vlim exist
  const bool tail_v = vlim < 128;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = wt * 128 + 32 * j + lr;
    const int64_t t = t0 + col;
    const bool tvalid = t < rows_valid;
    const int64_t trow = tvalid ? (row_map ? int64_t(row_map[t]) : t) : 0;
    const float tau = temp ? temp[trow] : temp_scalar;
    const float c = kLog2e / tau;

    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int vr = 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (!tail_v || vr < vlim) mx = fmaxf(mx, acc[i][j][r]);
      }
    Part p;
    p.m = mx * c;
    p.s = 0.0f;
    p.a = 0.0f;
    if (mx == kNegInf) {  // every value masked, or NaN values that fmaxf dropped
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int vr = 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
          if (vr < vlim && acc[i][j][r] != acc[i][j][r]) p.s = __builtin_nanf("");
        }
    } else if (!tail_v) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float d = __builtin_fmaf(acc[i][j][r], c, -p.m);
          const float e = exp2_hw(d);
          p.s += e;
          p.a = __builtin_fmaf(e, d, p.a);
        }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int vr = 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
          if (vr < vlim) {
            const float d = __builtin_fmaf(acc[i][j][r], c, -p.m);
            const float e = exp2_hw(d);
            p.s += e;
            p.a = __builtin_fmaf(e, d, p.a);
          }
        }
    }

    // the target's raw logit, if this lane holds it (exactly one lane in the grid does)
    if (tvalid) {
      const int64_t dv64 = targets[trow] - (v0 + wv * 128);
      if (dv64 >= 0 && dv64 < vlim && dv64 < 128) {
        const int dv = int(dv64);
        const int rr = dv & 31;
        if (((rr >> 2) & 1) == lh) {
          const int ii = dv >> 5;
          const int reg = (rr >> 3) * 4 + (rr & 3);
          float zv = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (i == ii && r == reg) zv = acc[i][j][r];
          zy_raw[t] = zv;
        }
      }
    }

    // merge the two half-waves (same column, other rows), then the two V waves
    Part q;
    q.m = shfl_xor_f(p.m, 32);
    q.s = shfl_xor_f(p.s, 32);
    q.a = shfl_xor_f(p.a, 32);
    p = merge(p, q);
    if (wv == 1 && lh == 0) {
      float* dst = red + (wt * 128 + 32 * j + lr) * 3;
      dst[0] = p.m;
      dst[1] = p.s;
      dst[2] = p.a;
    }
    __syncthreads();
    if (wv == 0 && lh == 0 && tvalid) {
      const float* src = red + (wt * 128 + 32 * j + lr) * 3;
      p = merge(p, Part{src[0], src[1], src[2]});
      partials[t * n_vtiles + vt] = make_float4(p.m, p.s, p.a, 0.0f);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(NT, 1) void fused_partials_kernel(
    const uint16_t* __restrict__ hidden, int64_t ld_h, const uint16_t* __restrict__ weight, int64_t ld_w,
    int64_t rows, int64_t H, int64_t V, const float* __restrict__ temp, float temp_scalar,
    const int64_t* __restrict__ targets, const int32_t* __restrict__ row_map, const int32_t* __restrict__ row_count,
    int n_vtiles, int n_ttiles, float4* __restrict__ partials, float* __restrict__ zy_raw) {
  const int nb = gridDim.x;  // a multiple of 8
  const int b = blockIdx.x;
  const int L = (b & 7) * (nb >> 3) + (b >> 3);
  if (L >= n_vtiles * n_ttiles) return;
  const int vt = L / n_ttiles;
  const int tt = L - vt * n_ttiles;
  const int64_t rows_valid = row_count ? int64_t(*row_count) : rows;
  const int64_t t0 = int64_t(tt) * BT;
  if (t0 >= rows_valid) return;
  const int64_t v0 = int64_t(vt) * BV;

  __shared__ uint4 As[2][BV * CH];
  __shared__ uint4 Bs[2][BT * CH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wv = w & 1;
  const int wt = w >> 1;

  // global -> LDS assignment: chunk idx = tid + NT*i -> (row r, chunk c)
  const uint16_t* a_src[LOADS];
  const uint16_t* b_src[LOADS];
  int lds_pos[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int idx = tid + NT * i;
    const int r = idx / CH;
    const int c = idx % CH;
    int64_t v = v0 + r;
    v = v < V ? v : V - 1;
    int64_t t = t0 + r;
    t = t < rows_valid ? t : rows_valid - 1;
    const int64_t hrow = row_map ? int64_t(row_map[t]) : t;
    a_src[i] = weight + v * ld_w + c * 8;
    b_src[i] = hidden + hrow * ld_h + c * 8;
    lds_pos[i] = swz(r, c);
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  uint4 ra[LOADS], rb[LOADS];
  // K-slice chunk validity (H is a multiple of 8; a slice may run past H)
  auto load_stage = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = (tid + NT * i) % CH;
      const bool ok = k0 + c * 8 < H;
      ra[i] = ok ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
      rb[i] = ok ? *reinterpret_cast<const uint4*>(b_src[i] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      As[buf][lds_pos[i]] = ra[i];
      Bs[buf][lds_pos[i]] = rb[i];
    }
  };

  load_stage(0);
  store_stage(0);
  __syncthreads();

  const int lr = lane & 31;  // row within a 32-row fragment
  const int lh = lane >> 5;  // which 8-wide K half of a 16-wide MFMA step
  int cur = 0;
  for (int64_t k0 = 0; k0 < H; k0 += BK) {
    const bool more = k0 + BK < H;
    if (more) load_stage(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wv * 128 + 32 * i + lr;
        af[i] = as_bf16x8(As[cur][swz(r, 2 * kk + lh)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wt * 128 + 32 * j + lr;
        bfr[j] = as_bf16x8(Bs[cur][swz(r, 2 * kk + lh)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) store_stage(cur ^ 1);
    __syncthreads();
    cur ^= 1;
  }

  tile_epilogue(acc, reinterpret_cast<float*>(&As[0][0]), v0, t0, vt, rows_valid, V, temp, temp_scalar, targets,
                row_map, n_vtiles, partials, zy_raw);
}


// ---------------------------------------------------------------------------
// Pipelined sweep (H a multiple of 32): the same tile, MFMA layout, swizzle
// and epilogue, but the K slices are brought into a 4-stage LDS ring by
// direct-to-LDS 16-byte loads issued three stages ahead (no staging
// registers).  Each stage lives in its own LDS array and the K loop is
// unrolled by 4, so the compiler can tell a stage being filled from the one
// being read and does not drain the loads before every LDS read.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }

constexpr int NSTAGE = 4;

struct Stage {
  uint4 a[BV * CH];
  uint4 b[BT * CH];
};
constexpr int DMA_PER_OP = BV * CH / NT;  // 16-byte loads per lane per operand per stage (4)
constexpr int DMA_PER_STAGE = 2 * DMA_PER_OP;

__global__ __launch_bounds__(NT, 1) void fused_partials_pipelined_kernel(
    const uint16_t* __restrict__ hidden, int64_t ld_h, const uint16_t* __restrict__ weight, int64_t ld_w,
    int64_t rows, int64_t H, int64_t V, const float* __restrict__ temp, float temp_scalar,
    const int64_t* __restrict__ targets, const int32_t* __restrict__ row_map, const int32_t* __restrict__ row_count,
    int n_vtiles, int n_ttiles, float4* __restrict__ partials, float* __restrict__ zy_raw) {
  const int nb = gridDim.x;  // a multiple of 8
  const int b = blockIdx.x;
  const int L = (b & 7) * (nb >> 3) + (b >> 3);
  if (L >= n_vtiles * n_ttiles) return;
  const int vt = L / n_ttiles;
  const int tt = L - vt * n_ttiles;
  const int64_t rows_valid = row_count ? int64_t(*row_count) : rows;
  const int64_t t0 = int64_t(tt) * BT;
  if (t0 >= rows_valid) return;
  const int64_t v0 = int64_t(vt) * BV;

  // one LDS object per ring slot (A and B tiles together): the compiler's
  // wait tracking tells the slot being filled from the one being read
  __shared__ Stage S0, S1, S2, S3;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wv = w & 1;
  const int wt = w >> 1;

  // Direct-to-LDS assignment: load i of wave w fills LDS chunks (4w + i) * 64 + lane,
  // i.e. row r = chunk / 4, physical slot chunk % 4, which holds logical K chunk
  // slot ^ ((r >> 1) & 3) of that row (the XOR swizzle the fragment reads undo).
  const uint16_t* ga[DMA_PER_OP];
  const uint16_t* gb[DMA_PER_OP];
#pragma unroll
  for (int i = 0; i < DMA_PER_OP; ++i) {
    const int p = (w * DMA_PER_OP + i) * 64 + lane;
    const int r = p >> 2;
    const int c = (p & 3) ^ ((r >> 1) & 3);
    int64_t v = v0 + r;
    v = v < V ? v : V - 1;
    int64_t t = t0 + r;
    t = t < rows_valid ? t : rows_valid - 1;
    const int64_t hrow = row_map ? int64_t(row_map[t]) : t;
    ga[i] = weight + v * ld_w + c * 8;
    gb[i] = hidden + hrow * ld_h + c * 8;
  }
  const int dma_off = w * DMA_PER_OP * 64;  // first chunk of this wave's loads

#define VS_DMA(St, k0)                                                                                   \
  do {                                                                                                   \
    _Pragma("unroll") for (int i_ = 0; i_ < DMA_PER_OP; ++i_) {                                          \
      __builtin_amdgcn_global_load_lds(ga[i_] + (k0), (lds_void_t*)(St.a + dma_off + i_ * 64), 16, 0, 0); \
      __builtin_amdgcn_global_load_lds(gb[i_] + (k0), (lds_void_t*)(St.b + dma_off + i_ * 64), 16, 0, 0); \
    }                                                                                                    \
  } while (0)

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int nk = int(H / BK);

#define VS_MMA(St)                                                              \
  do {                                                                          \
    bf16x8 fa[2][4], fb[2][4];                                                  \
    _Pragma("unroll") for (int kk = 0; kk < 2; ++kk) {                          \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                             \
        fa[kk][i] = as_bf16x8(St.a[swz(wv * 128 + 32 * i + lr, 2 * kk + lh)]);  \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                             \
        fb[kk][j] = as_bf16x8(St.b[swz(wt * 128 + 32 * j + lr, 2 * kk + lh)]);  \
    }                                                                           \
    _Pragma("unroll") for (int kk = 0; kk < 2; ++kk)                            \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                             \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                           \
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][i], fb[kk][j], acc[i][j], 0, 0, 0); \
  } while (0)

  // Main loop, whole groups of 4 stages.  Stage s: wait until this wave's
  // loads for stage s are done (the two younger stages may stay in flight),
  // barrier (every wave's loads for s are done, and every wave has finished
  // reading stage s-1), refill the slot of stage s-1 with stage s+3, compute
  // stage s.  The refill is unconditional (clamped to the last stage) so the
  // compiler's wait tracking stays exact.
#define VS_STEP(St, Sn, s)                                                   \
  {                                                                          \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * DMA_PER_STAGE));                \
    __builtin_amdgcn_s_barrier();                                            \
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");          \
    const int pf_ = (s) + 3 < nk ? (s) + 3 : nk - 1;                         \
    VS_DMA(Sn, int64_t(pf_) * BK);                                           \
    VS_MMA(St);                                                              \
  }

  VS_DMA(S0, 0);
  VS_DMA(S1, int64_t(1 < nk ? 1 : nk - 1) * BK);
  VS_DMA(S2, int64_t(2 < nk ? 2 : nk - 1) * BK);
  const int nk4 = nk & ~(NSTAGE - 1);
  for (int kt = 0; kt < nk4; kt += NSTAGE) {
    VS_STEP(S0, S3, kt)
    VS_STEP(S1, S0, kt + 1)
    VS_STEP(S2, S1, kt + 2)
    VS_STEP(S3, S2, kt + 3)
  }
  // leftover stages (nk % 4 of them) sit in slots 0..2 already
  const int rem = nk - nk4;
  if (rem > 0) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    VS_MMA(S0);
    if (rem > 1) VS_MMA(S1);
    if (rem > 2) VS_MMA(S2);
  }
#undef VS_STEP
#undef VS_MMA
#undef VS_DMA
  __syncthreads();
  tile_epilogue(acc, reinterpret_cast<float*>(&S0.a[0]), v0, t0, vt, rows_valid, V, temp, temp_scalar, targets,
                row_map, n_vtiles, partials, zy_raw);
}

__global__ void round_hidden_kernel(const float* __restrict__ h, int64_t ld, int64_t rows, int64_t H,
                                    uint16_t* __restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * H) return;
  const int64_t r = i / H;
  const int64_t k = i - r * H;
  const uint32_t u = __float_as_uint(h[r * ld + k]);
  uint16_t o;
  if ((u & 0x7fffffffu) > 0x7f800000u) {
    o = uint16_t((u >> 16) | 0x40u);  // quiet NaN
  } else {
    o = uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);  // nearest, ties to even
  }
  out[i] = o;
}

}  // namespace

int launch_fused_partials(const uint16_t* hidden, int64_t ld_hidden, const uint16_t* weight, int64_t ld_weight,
                          int64_t rows, int64_t H, int64_t V, const float* temp, float temp_scalar,
                          const int64_t* targets, const int32_t* row_map, const int32_t* row_count,
                          void* partials, float* zy_raw, void* stream) {
  const int n_vtiles = int((V + BV - 1) / BV);
  const int n_ttiles = int((rows + BT - 1) / BT);
  const int64_t tiles = int64_t(n_vtiles) * n_ttiles;
  if (tiles <= 0) return 0;
  const int64_t grid = (tiles + 7) / 8 * 8;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (H % BK == 0) {
    fused_partials_pipelined_kernel<<<dim3(unsigned(grid)), dim3(NT), 0, s>>>(
        hidden, ld_hidden, weight, ld_weight, rows, H, V, temp, temp_scalar, targets, row_map, row_count, n_vtiles,
        n_ttiles, static_cast<float4*>(partials), zy_raw);
  } else {
    fused_partials_kernel<<<dim3(unsigned(grid)), dim3(NT), 0, s>>>(
        hidden, ld_hidden, weight, ld_weight, rows, H, V, temp, temp_scalar, targets, row_map, row_count, n_vtiles,
        n_ttiles, static_cast<float4*>(partials), zy_raw);
  }
  return int(hipGetLastError());
}

int launch_round_hidden(const float* hidden, int64_t ld_hidden, int64_t rows, int64_t H, uint16_t* out,
                        void* stream) {
  const int64_t n = rows * H;
  if (n <= 0) return 0;
  round_hidden_kernel<<<dim3(unsigned((n + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      hidden, ld_hidden, rows, H, out);
  return int(hipGetLastError());
}

}  // namespace vs
