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
//   * K is swept in 32-wide slices staged through LDS with a 16-byte-chunk
//     XOR swizzle (conflict-free fragment reads);
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

// 16-byte chunk c of tile row r sits at slot c ^ g(r) of that row (rows are
// 64 bytes).  g(r) = (r >> 2) & 3 makes the fragment reads (32 consecutive
// rows, one chunk per half-wave) free of LDS bank conflicts; measured with the
// SQ_LDS_BANK_CONFLICT counter on gfx950 against the other candidate XOR
// patterns, which all leave 1.3-4 conflict cycles per ds_read_b128.
__device__ __forceinline__ int swz_g(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swz(int r, int c) { return r * CH + (c ^ swz_g(r)); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Workgroup -> tile order.  Workgroup ids are handed to the 8 XCDs round robin,
// so id b runs on XCD b % 8.  The vocabulary tiles are cut into bands of gv
// tiles and band g is served by XCD g % 8; inside a band the token tiles
// advance in blocks of kBlockT, the gv x kBlockT tiles of a block back to
// back, so one XCD's L2 holds the weight tiles of its band and the hidden
// tiles of its block while they are reused.  The grid is
// 8 * ceil(bands / 8) * gv * n_ttiles; ids past the last band do nothing.
// gv = 0 (fewer than 8 vocabulary tiles): plain order, vocabulary tile fastest.
constexpr int kBlockT = 8;
__host__ __device__ inline int band_width(int n_vtiles) {
  return n_vtiles < 8 ? 0 : n_vtiles < 32 ? n_vtiles / 8 : 4;
}
__host__ __device__ inline int64_t tile_grid(int64_t n_vtiles, int64_t n_ttiles, int gv) {
  if (gv == 0) return n_vtiles * n_ttiles;
  const int64_t bands = (n_vtiles + gv - 1) / gv;
  return 8 * ((bands + 7) / 8) * gv * n_ttiles;
}
__device__ __forceinline__ bool map_tile(int b, int n_vtiles, int n_ttiles, int gv, int& vt, int& tt) {
  if (gv == 0) {
    tt = b / n_vtiles;
    vt = b - tt * n_vtiles;
    return tt < n_ttiles;
  }
  const int x = b & 7;
  const int li = b >> 3;
  const int per_band = gv * n_ttiles;
  const int band_local = li / per_band;
  const int within = li - band_local * per_band;
  const int tb = within / (gv * kBlockT);
  const int r = within - tb * (gv * kBlockT);
  const int gt = n_ttiles - tb * kBlockT < kBlockT ? n_ttiles - tb * kBlockT : kBlockT;  // ragged last block
  const int vv = r / gt;
  vt = (band_local * 8 + x) * gv + vv;
  tt = tb * kBlockT + (r - vv * gt);
  return vt < n_vtiles;
}

// ---- epilogue: per token column, fold this tile's 256 vocabulary rows ----
// acc[i][j][r] holds vocabulary row  wv*128 + 32i + 8(r/4) + 4*lh + (r%4)
// and token column                   wt*128 + 32j + lr          (lr = lane & 31, lh = lane >> 5).
// Each lane folds its 64 rows of one column into (max, sum 2^(u-max), sum 2^(u-max)(u-max));
// the two half-waves and the two V-direction waves are merged, and one partial per
// (token, vocabulary tile) is written.  The lane holding the target id stores its raw logit.
// `red` is >= 3 KiB of LDS that no wave reads any more.

// The target id and temperature of the lane's 4 token columns.  They are
// loaded when the workgroup starts, so their latency hides behind the K loop
// instead of stalling each column of the epilogue between its barriers.
struct ColumnLoads {
  int64_t y[4];
  float tau[4];
};
__device__ __forceinline__ ColumnLoads load_columns(int64_t t0, int64_t rows_valid, const float* __restrict__ temp,
                                                    float temp_scalar, const int64_t* __restrict__ targets,
                                                    const int32_t* __restrict__ row_map) {
  const int lane = threadIdx.x & 63;
  const int wt = threadIdx.x >> 7;
  ColumnLoads cl;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t t = t0 + wt * 128 + 32 * j + (lane & 31);
    const int64_t trow = t < rows_valid ? (row_map ? int64_t(row_map[t]) : t) : 0;
    cl.y[j] = targets[trow];
    cl.tau[j] = temp ? temp[trow] : temp_scalar;
  }
  return cl;
}

// Fold the 64 accumulator values of one token column held by this lane into
// (max, sum 2^(u-max), sum 2^(u-max)(u-max)) in base-2 units, u = x * c.
// TAIL: only rows r with vr(r) < vlim exist (the ragged last vocabulary tile).
template <bool TAIL>
__device__ __forceinline__ Part fold_column(const f32x16& x0, const f32x16& x1, const f32x16& x2, const f32x16& x3,
                                            float c, int lh, int vlim) {
  const f32x16* xs[4] = {&x0, &x1, &x2, &x3};
  // opaque copy: keeps the compiler from hoisting the 64 row masks out of the
  // (rare) ragged branch into scalar registers shared by every column
  if (TAIL) asm volatile("" : "+v"(vlim));
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int vr = 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (!TAIL || vr < vlim) mx = fmaxf(mx, (*xs[i])[r]);
    }
  Part p;
  p.m = mx * c;
  p.s = 0.0f;
  p.a = 0.0f;
  if (mx == kNegInf) {  // every value masked or -inf, or NaN values that fmaxf dropped
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int vr = 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        if ((!TAIL || vr < vlim) && (*xs[i])[r] != (*xs[i])[r]) p.s = __builtin_nanf("");
      }
    return p;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int vr = 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (!TAIL || vr < vlim) {
        const float d = __builtin_fmaf((*xs[i])[r], c, -p.m);
        const float e = exp2_hw(d);
        p.s += e;
        p.a = __builtin_fmaf(e, d, p.a);
      }
    }
  return p;
}

__device__ __forceinline__ void tile_epilogue(f32x16 (&acc)[4][4], float* red, int64_t v0, int64_t t0, int vt,
                                              int64_t rows_valid, int64_t V, const ColumnLoads& cl, int n_vtiles,
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
  Part pj[4];  // per column, after the half-wave merge
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // the accumulators of the columns not folded yet stay in AGPRs until their turn
#pragma unroll
    for (int jj = j + 1; jj < 4; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+a"(acc[i][jj]));
    const int col = wt * 128 + 32 * j + lr;
    const int64_t t = t0 + col;
    const bool tvalid = t < rows_valid;
    const float c = kLog2e / cl.tau[j];

    // one uniform branch per wave: the unmasked fold is a plain max / exp
    // chain; only the ragged last vocabulary tile pays for per-row masks
    Part p;
    if (tail_v)
      p = fold_column<true>(acc[0][j], acc[1][j], acc[2][j], acc[3][j], c, lh, vlim);
    else
      p = fold_column<false>(acc[0][j], acc[1][j], acc[2][j], acc[3][j], c, lh, vlim);

    // the target's raw logit, if this lane holds it (exactly one lane in the grid does)
    if (tvalid) {
      const int64_t dv64 = cl.y[j] - (v0 + wv * 128);
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

    // merge the two half-waves (same column, other rows)
    Part q;
    q.m = shfl_xor_f(p.m, 32);
    q.s = shfl_xor_f(p.s, 32);
    q.a = shfl_xor_f(p.a, 32);
    pj[j] = merge(p, q);
  }
  // merge the two vocabulary waves: one LDS exchange and one barrier for all
  // four columns (no barrier between columns, so their folds overlap)
  if (wv == 1 && lh == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float* dst = red + (wt * 128 + 32 * j + lr) * 3;
      dst[0] = pj[j].m;
      dst[1] = pj[j].s;
      dst[2] = pj[j].a;
    }
  }
  __syncthreads();
  if (wv == 0 && lh == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = t0 + wt * 128 + 32 * j + lr;
      if (t < rows_valid) {
        const float* src = red + (wt * 128 + 32 * j + lr) * 3;
        const Part p = merge(pj[j], Part{src[0], src[1], src[2]});
        partials[t * n_vtiles + vt] = make_float4(p.m, p.s, p.a, 0.0f);
      }
    }
  }
}

// Epilogue modes of the sweep kernels.  The K loop is the same in every mode
// (C[m, n] = sum_k A[m, k] B[n, k], A the "weight" rows on M, B the "hidden"
// rows on N, both contiguous in K):
//   kEpiPartials  the softmax statistics above (the forward scoring op);
//   kEpiGrad      the logits' gradient of sum_t (a_t logprob_t + b_t H_t):
//                 dx = (a ([v = y] - p_v) - b p_v (ln p_v + H)) / tau, written
//                 as bf16 into G[t][v] (zeros in the padding columns up to
//                 v_pad, the K multiple of the GEMM that reads them);
//   kEpiStore     C[m][n] = acc, or += acc (fp32, n contiguous): a plain GEMM;
//   kEpiLogits    the logits themselves, rounded to bf16 (nearest even) into
//                 G[t][v] (0 in the columns from V up to the next multiple of 4).
enum { kEpiPartials = 0, kEpiGrad = 1, kEpiStore = 2, kEpiLogits = 3 };
struct EpiArgs {
  float4* partials;          // kEpiPartials
  float* zy_raw;
  const float* lse;          // kEpiGrad: the forward's outputs, per token row
  const float* entropy;
  const float* grad_logprob;  // nullable: 0
  const float* grad_entropy;  // nullable: 0
  uint16_t* g;               // [rows][ld_g]: column = vocabulary row of the sweep
  int64_t ld_g;
  int64_t v_begin;           // vocabulary id of the sweep's first row (the target test)
  int64_t v_pad;             // G's columns are zero-filled up to this
  uint16_t* gt;              // nullable: G^T [V][ld_gt] (64-wide sweep only), zeros in columns rows .. t_pad-1
  int64_t ld_gt;
  int64_t t_pad;
  float* c;                  // kEpiStore
  int64_t ldc;
  int accumulate;
};

// Two fp32 values as packed bf16, a in the low half: round to nearest even
// (one v_cvt_pk_bf16_f32; a NaN stays a NaN).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// The row data of the lane's 4 token columns for the gradient, loaded when
// the workgroup starts (their latency hides behind the K loop): base-2 scale,
// 1/tau, base-2 LSE, entropy, the two upstream gradients (0 on a bad row) and
// the target's row relative to the sweep's first row.
struct GradColumns {
  float c[4], inv_tau[4], l2[4], h[4], ga[4], gb[4];
  int64_t y[4];
};
__device__ __forceinline__ GradColumns load_grad_columns(int64_t t0, int64_t rows_valid, const float* __restrict__ temp,
                                                         float temp_scalar, const int64_t* __restrict__ targets,
                                                         const EpiArgs& ep) {
  const int lane = threadIdx.x & 63;
  const int wt = threadIdx.x >> 7;
  GradColumns g;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t t = t0 + wt * 128 + 32 * j + (lane & 31);
    const int64_t tr = t < rows_valid ? t : 0;
    const float tau = temp ? temp[tr] : temp_scalar;
    const float lse = ep.lse[tr];
    const int64_t y = targets[tr];
    float ga = ep.grad_logprob ? ep.grad_logprob[tr] : 0.0f;
    float gb = ep.grad_entropy ? ep.grad_entropy[tr] : 0.0f;
    float h = gb != 0.0f ? ep.entropy[tr] : 0.0f;
    if (!(t < rows_valid && tau_ok(tau) && lse > -__builtin_inff() && lse < __builtin_inff() && h == h && y >= 0)) {
      ga = 0.0f;  // no gradient through a bad row (or a column past the last row)
      gb = 0.0f;
      h = 0.0f;
    }
    g.c[j] = kLog2e / tau;
    g.inv_tau[j] = 1.0f / tau;
    g.l2[j] = lse * kLog2e;  // base-2 LSE
    g.h[j] = h;
    g.ga[j] = ga;
    g.gb[j] = gb;
    g.y[j] = y - ep.v_begin;
  }
  return g;
}

// The bf16 epilogues hand each lane's 8-byte pieces (4 consecutive vocabulary
// rows vb .. vb+3 of token column col, tile-relative) to a sink: DirectStore
// writes them to G [token][vocabulary row] (ld_g a multiple of 4), the staged
// form below collects the tile in LDS and writes whole rows.
struct DirectStore {
  static constexpr bool kAllColumns = false;  // the epilogue may skip columns past the last row
  uint16_t* g_tile;  // G + t0 * ld_g + v0
  int ldg;           // < 2^31 / 256 (checked at launch): tile offsets stay 32-bit
  __device__ __forceinline__ void operator()(int col, int vb, uint2 v, bool tvalid) const {
    if (tvalid) *reinterpret_cast<uint2*>(g_tile + col * ldg + vb) = v;
  }
};

// The tile as bf16 in the LDS of the K loop (free after its last barrier):
// part k holds token columns 64k .. 64k+63, one 512-byte row of 256 vocabulary
// rows each; 16-byte chunk c of row r sits at c ^ (r & 31), so the puts (32
// columns, one chunk) and the row reads (one row, 32 chunks) are both free
// of bank conflicts.  flush() writes rows r < trows, columns below lim (a
// multiple of 4): 16-byte stores where G's rows are 16-byte aligned (an
// 8-byte one for a half chunk), so each wave store covers two whole 512-byte
// rows where the direct pieces touch 32 rows; else 8-byte stores.
struct StagedStore {
  static constexpr bool kAllColumns = false;
  uint4 *p0, *p1, *p2, *p3;  // (selected, not indexed: an indexed array would be placed in LDS itself)
  __device__ __forceinline__ uint4* part(int k) const { return k == 0 ? p0 : k == 1 ? p1 : k == 2 ? p2 : p3; }
  __device__ __forceinline__ void operator()(int col, int vb, uint2 v, bool) const {
    uint4* row = part(col >> 6) + (col & 63) * 32;
    reinterpret_cast<uint2*>(row + ((vb >> 3) ^ (col & 31)))[(vb >> 2) & 1] = v;
  }
  __device__ __forceinline__ void flush(uint16_t* g_tile, int64_t ldg, int trows, int lim) const {
    const int c = threadIdx.x & 31;
    const int r0 = threadIdx.x >> 5;  // 8 rows per pass
    const bool wide = ((ldg & 7) | (reinterpret_cast<uintptr_t>(g_tile) & 15)) == 0;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int r = r0 + 8 * k;  // part k >> 3 holds it
      if (r < trows && 8 * c + 4 <= lim) {
        const uint4 v = part(k >> 3)[(r & 63) * 32 + (c ^ (r & 31))];
        uint16_t* dst = g_tile + r * ldg + 8 * c;
        if (wide && 8 * c + 8 <= lim) {
          *reinterpret_cast<uint4*>(dst) = v;
        } else {
          *reinterpret_cast<uint2*>(dst) = make_uint2(v.x, v.y);
          if (8 * c + 8 <= lim) *reinterpret_cast<uint2*>(dst + 4) = make_uint2(v.z, v.w);
        }
      }
    }
  }
};

// The gradient sink of the 64-wide sweep: G directly, and G^T through the
// K loop's LDS: each value goes as 2 bytes into an LDS tile [vocabulary row]
// [256 tokens] (part k: rows 64k .. 64k+63, 512 bytes each; 16-byte chunk c
// of row r at c ^ (((r >> 1) & 3) << 2), so the two rows of one put and the
// row reads of flush_t fall on distinct banks).
struct GradStore {
  static constexpr bool kAllColumns = true;  // every column (zeros past the last row) for G^T
  DirectStore g;
  uint4 *p0, *p1, *p2, *p3;
  __device__ __forceinline__ uint4* part(int k) const { return k == 0 ? p0 : k == 1 ? p1 : k == 2 ? p2 : p3; }
  __device__ __forceinline__ void operator()(int col, int vb, uint2 v, bool tvalid) const {
    g(col, vb, v, tvalid);
    const uint32_t w[2] = {v.x, v.y};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = vb + e;
      uint4* row = part(r >> 6) + (r & 63) * 32;
      uint16_t* dst = reinterpret_cast<uint16_t*>(row + ((col >> 3) ^ (((r >> 1) & 3) << 2))) + (col & 7);
      *dst = uint16_t(w[e >> 1] >> (16 * (e & 1)));
    }
  }
  // G^T rows r < nrows (vocabulary rows of the tile), token columns below ncols (a multiple of 8)
  __device__ __forceinline__ void flush_t(uint16_t* gt_tile, int64_t ld, int nrows, int ncols) const {
    const int c = threadIdx.x & 31;
    const int r0 = threadIdx.x >> 5;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int r = r0 + 8 * k;  // part k >> 3 holds it
      if (r < nrows && 8 * c < ncols)
        *reinterpret_cast<uint4*>(gt_tile + r * ld + 8 * c) = part(k >> 3)[(r & 63) * 32 + (c ^ (((r >> 1) & 3) << 2))];
    }
  }
};

// The gradient of the tile's logits into G (bf16, nearest even).  A row whose
// LSE is not finite (a BAD_INPUT row of the forward) gets a zero gradient.
template <class Sink>
__device__ __forceinline__ void grad_epilogue(f32x16 (&acc)[4][4], int64_t v0, int64_t t0, int64_t rows_valid,
                                              int64_t V, const GradColumns& gc, const EpiArgs& ep, const Sink& put) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wv = w & 1;
  const int wt = w >> 1;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  // tile-relative limits (32-bit): rows vr < nv exist, rows vr < np are written
  const int vrow0 = wv * 128 + 4 * lh;  // + 32 i + 8 q + e
  const int nv = int(V - v0 < BV ? V - v0 : BV);
  const int np = int(ep.v_pad - v0 < BV ? ep.v_pad - v0 : BV);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // the accumulators of the columns not written yet stay in AGPRs until their turn
#pragma unroll
    for (int jj = j + 1; jj < 4; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+a"(acc[i][jj]));
    const int col = wt * 128 + 32 * j + lr;
    const bool tvalid = t0 + col < rows_valid;
    const float c = gc.c[j], inv_tau = gc.inv_tau[j], l2 = gc.l2[j], h = gc.h[j], ga = gc.ga[j], gb = gc.gb[j];
    const int64_t yv = gc.y[j] - v0;
    const int yr = (yv >= 0 && yv < BV) ? int(yv) : -1;  // the target's tile-relative row
    const bool live = tvalid && (ga != 0.0f || gb != 0.0f);  // else dx = 0
    if (!Sink::kAllColumns && !tvalid) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int vb = vrow0 + 32 * i + 8 * q;  // rows vb .. vb+3 of the tile
        if (vb >= np) continue;
        float dx[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dx[e] = 0.0f;
          if (live && vb + e < nv) {
            const float d2 = __builtin_fmaf(acc[i][j][4 * q + e], c, -l2);
            const float pv = exp2_hw(d2);
            float dz = -pv * __builtin_fmaf(gb, __builtin_fmaf(d2, kLn2, h), ga);
            if (vb + e == yr) dz += ga;
            dx[e] = dz * inv_tau;
          }
        }
        put(col, vb, make_uint2(pack_bf16_rne(dx[0], dx[1]), pack_bf16_rne(dx[2], dx[3])), tvalid);
      }
  }
}

// The tile's logits as bf16 into G [token][vocabulary row], in pieces of 4
// consecutive vocabulary rows (0 past V).
template <class Sink>
__device__ __forceinline__ void logits_epilogue(f32x16 (&acc)[4][4], int64_t v0, int64_t t0, int64_t rows_valid,
                                                int64_t V, const Sink& put) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wv = w & 1;
  const int wt = w >> 1;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int vrow0 = wv * 128 + 4 * lh;  // + 32 i + 8 q + e
  const int nv = int(V - v0 < BV ? V - v0 : BV);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int jj = j + 1; jj < 4; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+a"(acc[i][jj]));
    const int col = wt * 128 + 32 * j + lr;
    if (t0 + col >= rows_valid) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int vb = vrow0 + 32 * i + 8 * q;
        if (vb >= nv) continue;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = vb + e < nv ? acc[i][j][4 * q + e] : 0.0f;
        put(col, vb, make_uint2(pack_bf16_rne(x[0], x[1]), pack_bf16_rne(x[2], x[3])), true);
      }
  }
}

// C[m][n] (+)= acc for the rows m < M and columns n < N of the tile.
__device__ __forceinline__ void store_epilogue(f32x16 (&acc)[4][4], int64_t m0, int64_t n0, int64_t N, int64_t M,
                                               const EpiArgs& ep) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wv = w & 1;
  const int wt = w >> 1;
  const int lr = lane & 31;
  const int lh = lane >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int jj = j + 1; jj < 4; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+a"(acc[i][jj]));
    const int64_t n = n0 + wt * 128 + 32 * j + lr;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wv * 128 + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (m < M) {
          float* dst = ep.c + m * ep.ldc + n;
          *dst = ep.accumulate ? *dst + acc[i][j][r] : acc[i][j][r];
        }
      }
  }
}

template <int MODE>
__global__ __launch_bounds__(NT, 1) void fused_partials_kernel(
    const uint16_t* __restrict__ hidden, int64_t ld_h, const uint16_t* __restrict__ weight, int64_t ld_w,
    int64_t rows, int64_t H, int64_t V, const float* __restrict__ temp, float temp_scalar,
    const int64_t* __restrict__ targets, const int32_t* __restrict__ row_map, const int32_t* __restrict__ row_count,
    int n_vtiles, int n_ttiles, int gv, EpiArgs ep) {
  int vt, tt;
  if (!map_tile(int(blockIdx.x), n_vtiles, n_ttiles, gv, vt, tt)) return;
  const int64_t rows_valid = row_count ? int64_t(*row_count) : rows;
  const int64_t t0 = int64_t(tt) * BT;
  if (t0 >= rows_valid) return;
  const int64_t v0 = int64_t(vt) * BV;

  __shared__ uint4 As[2][BV * CH];
  __shared__ uint4 Bs[2][BT * CH];
  ColumnLoads cl{};
  GradColumns gcol{};
  if (MODE == kEpiPartials) cl = load_columns(t0, rows_valid, temp, temp_scalar, targets, row_map);
  if (MODE == kEpiGrad) gcol = load_grad_columns(t0, rows_valid, temp, temp_scalar, targets, ep);

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

  if constexpr (MODE == kEpiPartials)
    tile_epilogue(acc, reinterpret_cast<float*>(&As[0][0]), v0, t0, vt, rows_valid, V, cl, n_vtiles, ep.partials,
                  ep.zy_raw);
  else if constexpr (MODE == kEpiGrad)
    grad_epilogue(acc, v0, t0, rows_valid, V, gcol, ep, DirectStore{ep.g + t0 * ep.ld_g + v0, int(ep.ld_g)});
  else if constexpr (MODE == kEpiLogits)
    logits_epilogue(acc, v0, t0, rows_valid, V, DirectStore{ep.g + t0 * ep.ld_g + v0, int(ep.ld_g)});
  else
    store_epilogue(acc, v0, t0, rows_valid, V, ep);
}


// ---------------------------------------------------------------------------
// Pipelined sweep (H a multiple of 32): the same tile, MFMA layout, swizzle
// and epilogue, but the K slices are brought into a 4-slot LDS ring by
// direct-to-LDS 16-byte loads issued three stages ahead (no staging
// registers, no VGPR round trip).
//   * Each ring slot is its own pair of LDS arrays and the K loop is unrolled
//     by 4, so the compiler's wait tracking tells the slot being filled from
//     the slots being read and never drains the loads before an LDS read.
//   * BUF: the loads are buffer loads against one resource per operand tile,
//     with a 32-bit per-lane byte offset and the K offset in a scalar
//     register (half the address VGPRs and VALU work of 64-bit pointers).
//     Used when a 256-row operand tile spans less than 2 GiB and the hidden
//     rows are not gathered; otherwise the loads take 64-bit pointers.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediates: "at most vm vector-memory and lgkm LDS operations
// outstanding" (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14); }
constexpr int vmcnt_imm(int n) { return waitcnt_imm(n, 15); }
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;

constexpr int NSTAGE = 4;
constexpr int DMA_PER_OP = BV * CH / NT;  // 16-byte loads per lane per operand per stage (4)
constexpr int DMA_PER_STAGE = 2 * DMA_PER_OP;
// dword 3 of a raw buffer resource on gfx9-class parts: 32-bit data format, no swizzle
constexpr int kBufferFlags = 0x00020000;

template <bool BUF, int REM, int MODE>
__global__ __launch_bounds__(NT, 1) void fused_partials_pipelined_kernel(
    const uint16_t* __restrict__ hidden, int64_t ld_h, const uint16_t* __restrict__ weight, int64_t ld_w,
    int64_t rows, int64_t H, int64_t V, const float* __restrict__ temp, float temp_scalar,
    const int64_t* __restrict__ targets, const int32_t* __restrict__ row_map, const int32_t* __restrict__ row_count,
    int n_vtiles, int n_ttiles, int gv, EpiArgs ep) {
  int vt, tt;
  if (!map_tile(int(blockIdx.x), n_vtiles, n_ttiles, gv, vt, tt)) return;
  const int64_t rows_valid = row_count ? int64_t(*row_count) : rows;
  const int64_t t0 = int64_t(tt) * BT;
  if (t0 >= rows_valid) return;
  const int64_t v0 = int64_t(vt) * BV;

  __shared__ uint4 A0[BV * CH], A1[BV * CH], A2[BV * CH], A3[BV * CH];
  __shared__ uint4 B0[BT * CH], B1[BT * CH], B2[BT * CH], B3[BT * CH];
  ColumnLoads cl{};
  GradColumns gcol{};
  if (MODE == kEpiPartials) cl = load_columns(t0, rows_valid, temp, temp_scalar, targets, BUF ? nullptr : row_map);
  if (MODE == kEpiGrad) gcol = load_grad_columns(t0, rows_valid, temp, temp_scalar, targets, ep);
  // slot indices are compile-time constants after unrolling
  auto SA = [&](int i) -> uint4* { return i == 0 ? A0 : i == 1 ? A1 : i == 2 ? A2 : A3; };
  auto SB = [&](int i) -> uint4* { return i == 0 ? B0 : i == 1 ? B1 : i == 2 ? B2 : B3; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wv = w & 1;
  const int wt = w >> 1;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index, in a scalar register
  const int64_t vrows = V - v0 < BV ? V - v0 : BV;
  const int64_t trows = rows_valid - t0 < BT ? rows_valid - t0 : BT;

  // Load i of wave w fills LDS chunk p = (4w + i) * 64 + lane: tile row r = p / 4,
  // physical slot p % 4, which holds logical K chunk (p % 4) ^ g(r) of that row.
  // Rows past the tile's end re-read the last row (their results are masked).
  uint32_t oa[DMA_PER_OP], ob[DMA_PER_OP];      // BUF: byte offsets inside the tile
  const uint16_t* ga[DMA_PER_OP];               // otherwise: pointers
  const uint16_t* gb[DMA_PER_OP];
#pragma unroll
  for (int i = 0; i < DMA_PER_OP; ++i) {
    const int p = (w * DMA_PER_OP + i) * 64 + lane;
    const int r = p >> 2;
    const int c = (p & 3) ^ swz_g(r);
    const int64_t rv = r < vrows ? r : vrows - 1;
    const int64_t rt = r < trows ? r : trows - 1;
    if (BUF) {
      oa[i] = uint32_t((rv * ld_w + c * 8) * 2);
      ob[i] = uint32_t((rt * ld_h + c * 8) * 2);
    } else {
      const int64_t hrow = row_map ? int64_t(row_map[t0 + rt]) : t0 + rt;
      ga[i] = weight + (v0 + rv) * ld_w + c * 8;
      gb[i] = hidden + hrow * ld_h + c * 8;
    }
  }
  // (unused, and dropped by the compiler, when !BUF)
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(weight + v0 * ld_w), (short)0, int(BUF ? vrows * ld_w * 2 : 0), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(hidden + t0 * ld_h), (short)0, int(BUF ? trows * ld_h * 2 : 0), kBufferFlags);
  auto dma = [&](int slot, int64_t k0) {
    if (BUF) {
      const uint32_t so = uint32_t(k0 * 2);
#pragma unroll
      for (int i = 0; i < DMA_PER_OP; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)(SA(slot) + (wu * DMA_PER_OP + i) * 64), 16,
                                                 oa[i], so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lds_void_t*)(SB(slot) + (wu * DMA_PER_OP + i) * 64), 16,
                                                 ob[i], so, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < DMA_PER_OP; ++i) {
        __builtin_amdgcn_global_load_lds(ga[i] + k0, (lds_void_t*)(SA(slot) + (wu * DMA_PER_OP + i) * 64), 16, 0,
                                         0);
        __builtin_amdgcn_global_load_lds(gb[i] + k0, (lds_void_t*)(SB(slot) + (wu * DMA_PER_OP + i) * 64), 16, 0,
                                         0);
      }
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int lr = lane & 31;
  const int lh = lane >> 5;
  typedef bf16x8 Frags[2][4];
  auto read_slot = [&](int slot, Frags& fa, Frags& fb) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[kk][i] = as_bf16x8(SA(slot)[swz(wv * 128 + 32 * i + lr, 2 * kk + lh)]);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[kk][j] = as_bf16x8(SB(slot)[swz(wt * 128 + 32 * j + lr, 2 * kk + lh)]);
    }
  };
  auto mma = [&](const Frags& fa, const Frags& fb) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][i], fb[kk][j], acc[i][j], 0, 0, 0);
  };
  // barrier + "LDS reads stay after it"
  auto bar = [&]() {
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  const int nk = int(H / BK);
  // prologue: stages 0..3 into slots 0..3 (clamped to the last stage), then
  // the fragments of stage 0 into register set 0
#pragma unroll
  for (int s = 0; s < NSTAGE; ++s) dma(s, int64_t(s < nk ? s : nk - 1) * BK);
  Frags fa0, fb0, fa1, fb1;
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((NSTAGE - 1) * DMA_PER_STAGE));
  bar();
  read_slot(0, fa0, fb0);
  // Stage s lives in slot s % 4, and during step s-1 its fragments move to
  // register set s % 2.  Step s:
  //   1. wait until this wave's loads for stage s+1 have landed (s+2 and s+3
  //      stay in flight) and its reads of slot s % 4 are done;
  //   2. barrier: every wave's loads for s+1 are in LDS, and no wave reads
  //      slot s % 4 any more;
  //   3. issue, interleaved: the 32 MFMAs of stage s from registers, the 16
  //      fragment reads of stage s+1, and the refill of slot s % 4 with stage
  //      s+4 (one read per MFMA pair, one load per four MFMAs).
  // With one wave per SIMD the reads only overlap the MFMAs when they are
  // spread among them: a burst of reads stalls issue until LDS drains it.
  // Loads are unconditional (clamped to the last stage), so the wait counts
  // stay exact; the refill's slot is a separate LDS array from the one being
  // read, so the compiler's wait tracking never drains the loads before a
  // read.  The last step's read of stage nk re-reads a clamped duplicate.
  auto step = [&](int u, int s, Frags& fa_cur, Frags& fb_cur, Frags& fa_nxt, Frags& fb_nxt) {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm((NSTAGE - 2) * DMA_PER_STAGE, 0));
    bar();
    read_slot((u + 1) % NSTAGE, fa_nxt, fb_nxt);
    const int pf = s + NSTAGE < nk ? s + NSTAGE : nk - 1;
    dma(u, int64_t(pf) * BK);
    mma(fa_cur, fb_cur);
#pragma unroll
    for (int q = 0; q < DMA_PER_STAGE; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  const int nk4 = nk - REM;
  for (int kt = 0; kt < nk4; kt += NSTAGE) {
    step(0, kt + 0, fa0, fb0, fa1, fb1);
    step(1, kt + 1, fa1, fb1, fa0, fb0);
    step(2, kt + 2, fa0, fb0, fa1, fb1);
    step(3, kt + 3, fa1, fb1, fa0, fb0);
  }
  // the REM = nk % 4 leftover stages: slots 0 .. REM-1, register sets 0, 1, 0
  if (REM > 0) step(0, nk4 + 0, fa0, fb0, fa1, fb1);
  if (REM > 1) step(1, nk4 + 1, fa1, fb1, fa0, fb0);
  if (REM > 2) step(2, nk4 + 2, fa0, fb0, fa1, fb1);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // clamped duplicate refills may still be landing
  __syncthreads();
  if constexpr (MODE == kEpiPartials)
    tile_epilogue(acc, reinterpret_cast<float*>(&A0[0]), v0, t0, vt, rows_valid, V, cl, n_vtiles, ep.partials,
                  ep.zy_raw);
  else if constexpr (MODE == kEpiGrad)
    grad_epilogue(acc, v0, t0, rows_valid, V, gcol, ep, DirectStore{ep.g + t0 * ep.ld_g + v0, int(ep.ld_g)});
  else if constexpr (MODE == kEpiLogits)
    logits_epilogue(acc, v0, t0, rows_valid, V, DirectStore{ep.g + t0 * ep.ld_g + v0, int(ep.ld_g)});
  else
    store_epilogue(acc, v0, t0, rows_valid, V, ep);
}

// ---------------------------------------------------------------------------
// Wide-stage sweep (H a multiple of 64): the same tile, MFMA layout and
// epilogue, with the K slices staged 64 wide, so each tile row's slice is one
// whole 128-byte line.  With 32-wide slices every refill load touches half of
// 16 lines and the other half is fetched again one stage later; the load path
// then costs ~20% of the loop.  Here each 16-byte-per-lane load covers 8 rows
// x 128 bytes.
//   * Ring: 2 slots x (A 32 KiB + B 32 KiB).  Row r of a slot is 8 chunks of
//     16 bytes; chunk c sits at c ^ g8(r), g8(r) = (r >> 1) & 7, which keeps
//     the fragment reads (32 rows, one chunk per half-wave; the LDS serves 16
//     lanes per pass over its 256-byte bank row) free of bank conflicts.
//   * Each 64-wide stage is two 32-wide sub-steps of 32 MFMAs.  Fragments of
//     the next sub-step are read into the other register set while the
//     current sub-step's MFMAs run, one read per MFMA pair.
//   * One barrier per stage, at its second sub-step: the next stage has
//     landed, and no wave reads the current slot any more, so its refill
//     (stage S+2) is issued right there, one load per MFMA pair.
// ---------------------------------------------------------------------------
constexpr int BK2 = 64;
constexpr int CH2 = BK2 / 8;                  // 16-byte chunks per row per stage (8)
constexpr int DMA2_PER_OP = BV * CH2 / NT;    // loads per lane per operand per stage (8)
constexpr int DMA2_PER_STAGE = 2 * DMA2_PER_OP;
__device__ __forceinline__ int swz8(int r, int c) { return r * CH2 + (c ^ ((r >> 1) & 7)); }

template <bool BUF, int REM, int MODE>
__global__ __launch_bounds__(NT, 1) void fused_partials_wide_kernel(
    const uint16_t* __restrict__ hidden, int64_t ld_h, const uint16_t* __restrict__ weight, int64_t ld_w,
    int64_t rows, int64_t H, int64_t V, const float* __restrict__ temp, float temp_scalar,
    const int64_t* __restrict__ targets, const int32_t* __restrict__ row_map, const int32_t* __restrict__ row_count,
    int n_vtiles, int n_ttiles, int gv, EpiArgs ep) {
  int vt, tt;
  if (!map_tile(int(blockIdx.x), n_vtiles, n_ttiles, gv, vt, tt)) return;
  const int64_t rows_valid = row_count ? int64_t(*row_count) : rows;
  const int64_t t0 = int64_t(tt) * BT;
  if (t0 >= rows_valid) return;
  const int64_t v0 = int64_t(vt) * BV;

  __shared__ uint4 A0[BV * CH2], A1[BV * CH2];
  __shared__ uint4 B0[BT * CH2], B1[BT * CH2];
  auto SA = [&](int i) -> uint4* { return i == 0 ? A0 : A1; };
  auto SB = [&](int i) -> uint4* { return i == 0 ? B0 : B1; };
  ColumnLoads cl{};
  GradColumns gcol{};
  if (MODE == kEpiPartials) cl = load_columns(t0, rows_valid, temp, temp_scalar, targets, BUF ? nullptr : row_map);
  if (MODE == kEpiGrad) gcol = load_grad_columns(t0, rows_valid, temp, temp_scalar, targets, ep);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wv = w & 1;
  const int wt = w >> 1;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int64_t vrows = V - v0 < BV ? V - v0 : BV;
  const int64_t trows = rows_valid - t0 < BT ? rows_valid - t0 : BT;

  // Load i of wave w fills LDS chunk p = (8w + i) * 64 + lane: row r = p / 8,
  // physical chunk p % 8, which holds logical chunk (p % 8) ^ g8(r).  Rows
  // past the tile's end re-read the last row (their results are masked).
  uint32_t oa[DMA2_PER_OP], ob[DMA2_PER_OP];
  const uint16_t* ga[DMA2_PER_OP];
  const uint16_t* gb[DMA2_PER_OP];
#pragma unroll
  for (int i = 0; i < DMA2_PER_OP; ++i) {
    const int p = (w * DMA2_PER_OP + i) * 64 + lane;
    const int r = p >> 3;
    const int c = (p & 7) ^ ((r >> 1) & 7);
    const int64_t rv = r < vrows ? r : vrows - 1;
    const int64_t rt = r < trows ? r : trows - 1;
    if (BUF) {
      oa[i] = uint32_t((rv * ld_w + c * 8) * 2);
      ob[i] = uint32_t((rt * ld_h + c * 8) * 2);
    } else {
      const int64_t hrow = row_map ? int64_t(row_map[t0 + rt]) : t0 + rt;
      ga[i] = weight + (v0 + rv) * ld_w + c * 8;
      gb[i] = hidden + hrow * ld_h + c * 8;
    }
  }
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(weight + v0 * ld_w), (short)0, int(BUF ? vrows * ld_w * 2 : 0), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(hidden + t0 * ld_h), (short)0, int(BUF ? trows * ld_h * 2 : 0), kBufferFlags);
  auto dma = [&](int slot, int64_t k0) {
    if (BUF) {
      const uint32_t so = uint32_t(k0 * 2);
#pragma unroll
      for (int i = 0; i < DMA2_PER_OP; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)(SA(slot) + (wu * DMA2_PER_OP + i) * 64), 16,
                                                 oa[i], so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lds_void_t*)(SB(slot) + (wu * DMA2_PER_OP + i) * 64), 16,
                                                 ob[i], so, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < DMA2_PER_OP; ++i) {
        __builtin_amdgcn_global_load_lds(ga[i] + k0, (lds_void_t*)(SA(slot) + (wu * DMA2_PER_OP + i) * 64), 16, 0,
                                         0);
        __builtin_amdgcn_global_load_lds(gb[i] + k0, (lds_void_t*)(SB(slot) + (wu * DMA2_PER_OP + i) * 64), 16, 0,
                                         0);
      }
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int lr = lane & 31;
  const int lh = lane >> 5;
  typedef bf16x8 Frags[2][4];
  // fragments of half h (K 32h .. 32h+31) of the stage in `slot`
  auto read_half = [&](int slot, int h, Frags& fa, Frags& fb) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[kk][i] = as_bf16x8(SA(slot)[swz8(wv * 128 + 32 * i + lr, 4 * h + 2 * kk + lh)]);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[kk][j] = as_bf16x8(SB(slot)[swz8(wt * 128 + 32 * j + lr, 4 * h + 2 * kk + lh)]);
    }
  };
  auto mma = [&](const Frags& fa, const Frags& fb) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][i], fb[kk][j], acc[i][j], 0, 0, 0);
  };
  auto bar = [&]() {
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  const int nk = int(H / BK2);
  // prologue: stages 0 and 1 (clamped) into slots 0 and 1; half 0 of stage 0 into register set 0
  dma(0, 0);
  dma(1, int64_t(1 < nk ? 1 : 0) * BK2);
  Frags fa0, fb0, fa1, fb1;
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(DMA2_PER_STAGE));
  bar();
  read_half(0, 0, fa0, fb0);
  // Stage S (slot S % 2), sub-step 0: read half 1 of S into set 1, MFMAs of
  // half 0 (set 0).  Sub-step 1: wait until this wave's loads of stage S+1
  // (the only ones in flight) and its reads of slot S % 2 are done; barrier;
  // read half 0 of S+1 into set 0, refill slot S % 2 with stage S+2 (clamped
  // to the last stage: unconditional loads keep the wait counts exact), MFMAs
  // of half 1 (set 1).  The refill's slot is a separate LDS array from the one
  // being read, so the compiler's wait tracking never drains the loads before
  // a read.  The last stage's read of stage nk re-reads a clamped duplicate.
  auto stage = [&](int u, int S) {
    read_half(u, 1, fa1, fb1);
    mma(fa0, fb0);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    bar();
    read_half(u ^ 1, 0, fa0, fb0);
    const int pf = S + 2 < nk ? S + 2 : nk - 1;
    dma(u, int64_t(pf) * BK2);
    mma(fa1, fb1);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  const int nk2 = nk - REM;
  for (int S = 0; S < nk2; S += 2) {
    stage(0, S);
    stage(1, S + 1);
  }
  if (REM) stage(0, nk2);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // clamped duplicate refills may still be landing
  __syncthreads();
  if constexpr (MODE == kEpiPartials)
    tile_epilogue(acc, reinterpret_cast<float*>(&A0[0]), v0, t0, vt, rows_valid, V, cl, n_vtiles, ep.partials,
                  ep.zy_raw);
  else if constexpr (MODE == kEpiGrad) {
    const DirectStore gd{ep.g + t0 * ep.ld_g + v0, int(ep.ld_g)};
    if constexpr (BUF && REM == 0) {  // G^T too (the other forms have no registers to spare for it)
      const GradStore st{gd, A0, A1, B0, B1};
      grad_epilogue(acc, v0, t0, rows_valid, V, gcol, ep, st);
      __syncthreads();
      st.flush_t(ep.gt + v0 * ep.ld_gt + t0, ep.ld_gt, int(vrows), int(ep.t_pad - t0 < BT ? ep.t_pad - t0 : BT));
    } else {
      grad_epilogue(acc, v0, t0, rows_valid, V, gcol, ep, gd);
    }
  } else if constexpr (MODE == kEpiLogits) {
    const StagedStore st{A0, A1, B0, B1};
    logits_epilogue(acc, v0, t0, rows_valid, V, st);
    __syncthreads();
    st.flush(ep.g + t0 * ep.ld_g + v0, ep.ld_g, int(trows), (int(vrows) + 3) & ~3);
  } else
    store_epilogue(acc, v0, t0, rows_valid, V, ep);
}

// dst[c][r] = src[r][c] for c < C, r < R_pad (0 for r >= R), by 64 x 64
// tiles through LDS.  A thread moves 16 consecutive values (two 16-byte
// accesses where the row's alignment and extent allow, else one value at a
// time) on both sides.
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t* __restrict__ src, int64_t ld_s, int64_t R,
                                                            int64_t C, uint16_t* __restrict__ dst, int64_t ld_d,
                                                            int64_t R_pad) {
  __shared__ uint16_t tile[64][72];  // row stride 144 B: 16-byte aligned, rows spread over the banks
  const int64_t r0 = int64_t(blockIdx.y) * 64, c0 = int64_t(blockIdx.x) * 64;
  const int a = threadIdx.x >> 2, b = (threadIdx.x & 3) * 16;  // row a, columns b .. b+15 of the tile
  {
    const int64_t r = r0 + a, c = c0 + b;
    uint4 v[2];
    uint16_t* h = reinterpret_cast<uint16_t*>(v);
    const uint16_t* p = src + r * ld_s + c;
    if (r < R && c + 16 <= C && ((reinterpret_cast<uintptr_t>(p) & 15) == 0)) {
      v[0] = reinterpret_cast<const uint4*>(p)[0];
      v[1] = reinterpret_cast<const uint4*>(p)[1];
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) h[k] = (r < R && c + k < C) ? p[k] : uint16_t(0);
    }
    *reinterpret_cast<uint4*>(&tile[a][b]) = v[0];
    *reinterpret_cast<uint4*>(&tile[a][b + 8]) = v[1];
  }
  __syncthreads();
  {
    const int64_t c = c0 + a, r = r0 + b;  // output row c, its columns r .. r+15
    if (c >= C || r >= R_pad) return;
    uint4 v[2];
    uint16_t* h = reinterpret_cast<uint16_t*>(v);
#pragma unroll
    for (int k = 0; k < 16; ++k) h[k] = tile[b + k][a];
    uint16_t* p = dst + c * ld_d + r;
    if (r + 16 <= R_pad && ((reinterpret_cast<uintptr_t>(p) & 15) == 0)) {
      reinterpret_cast<uint4*>(p)[0] = v[0];
      reinterpret_cast<uint4*>(p)[1] = v[1];
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (r + k < R_pad) p[k] = h[k];
    }
  }
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

namespace {

// One sweep over every (vocabulary tile, token tile) of weight rows [0, V) x
// hidden rows [0, rows), K = H, in the epilogue mode MODE.
template <int MODE>
int launch_sweep(const uint16_t* hidden, int64_t ld_hidden, const uint16_t* weight, int64_t ld_weight, int64_t rows,
                 int64_t H, int64_t V, const float* temp, float temp_scalar, const int64_t* targets,
                 const int32_t* row_map, const int32_t* row_count, const EpiArgs& ep, void* stream) {
  const int64_t n_vtiles = (V + BV - 1) / BV;
  const int64_t n_ttiles = (rows + BT - 1) / BT;
  if (n_vtiles <= 0 || n_ttiles <= 0) return 0;
  if (n_vtiles > 0x7FFFFFFF || n_ttiles > 0x7FFFFFFF) return int(hipErrorInvalidConfiguration);
  const int gv = band_width(int(n_vtiles));
  const int64_t grid = tile_grid(n_vtiles, n_ttiles, gv);
  if (grid > 0x7FFFFFFF) return int(hipErrorInvalidConfiguration);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 g{unsigned(grid)}, b{unsigned(NT)};
  const int nv = int(n_vtiles), nt = int(n_ttiles);
  // buffer offsets are 32-bit: a 256-row tile of either operand must span < 2 GiB
  const bool buf_ok = !row_map && int64_t(BV) * ld_weight * 2 <= 0x7FFFFFFF && int64_t(BT) * ld_hidden * 2 <= 0x7FFFFFFF;
  if (H % BK2 == 0) {
    const int rem = int((H / BK2) % 2);
#define VS_LAUNCH_WIDE(B, R)                                                                                       \
  fused_partials_wide_kernel<B, R, MODE><<<g, b, 0, s>>>(hidden, ld_hidden, weight, ld_weight, rows, H, V, temp,    \
                                                         temp_scalar, targets, row_map, row_count, nv, nt, gv, ep)
    switch (rem + (buf_ok ? 0 : 2)) {
      case 0: VS_LAUNCH_WIDE(true, 0); break;
      case 1: VS_LAUNCH_WIDE(true, 1); break;
      case 2: VS_LAUNCH_WIDE(false, 0); break;
      default: VS_LAUNCH_WIDE(false, 1); break;
    }
#undef VS_LAUNCH_WIDE
  } else if (H % BK == 0) {
    const int rem = int((H / BK) % NSTAGE);
#define VS_LAUNCH_PIPELINED(B, R)                                                                                  \
  fused_partials_pipelined_kernel<B, R, MODE><<<g, b, 0, s>>>(hidden, ld_hidden, weight, ld_weight, rows, H, V,     \
                                                              temp, temp_scalar, targets, row_map, row_count, nv,  \
                                                              nt, gv, ep)
    switch (rem + (buf_ok ? 0 : 4)) {
      case 0: VS_LAUNCH_PIPELINED(true, 0); break;
      case 1: VS_LAUNCH_PIPELINED(true, 1); break;
      case 2: VS_LAUNCH_PIPELINED(true, 2); break;
      case 3: VS_LAUNCH_PIPELINED(true, 3); break;
      case 4: VS_LAUNCH_PIPELINED(false, 0); break;
      case 5: VS_LAUNCH_PIPELINED(false, 1); break;
      case 6: VS_LAUNCH_PIPELINED(false, 2); break;
      default: VS_LAUNCH_PIPELINED(false, 3); break;
    }
#undef VS_LAUNCH_PIPELINED
  } else {
    fused_partials_kernel<MODE><<<g, b, 0, s>>>(hidden, ld_hidden, weight, ld_weight, rows, H, V, temp, temp_scalar,
                                                targets, row_map, row_count, nv, nt, gv, ep);
  }
  return int(hipGetLastError());
}

}  // namespace

int launch_fused_partials(const uint16_t* hidden, int64_t ld_hidden, const uint16_t* weight, int64_t ld_weight,
                          int64_t rows, int64_t H, int64_t V, const float* temp, float temp_scalar,
                          const int64_t* targets, const int32_t* row_map, const int32_t* row_count,
                          void* partials, float* zy_raw, void* stream) {
  EpiArgs ep{};
  ep.partials = static_cast<float4*>(partials);
  ep.zy_raw = zy_raw;
  return launch_sweep<kEpiPartials>(hidden, ld_hidden, weight, ld_weight, rows, H, V, temp, temp_scalar, targets,
                                    row_map, row_count, ep, stream);
}

bool fused_grad_writes_transpose(int64_t H, int64_t ld_hidden, int64_t ld_weight) {
  // the 64-wide sweep with an even stage count and 32-bit buffer offsets (as launch_sweep picks it)
  return H % (2 * BK2) == 0 && int64_t(BV) * ld_weight * 2 <= 0x7FFFFFFF && int64_t(BT) * ld_hidden * 2 <= 0x7FFFFFFF;
}

int launch_fused_grad(const uint16_t* hidden, int64_t ld_hidden, const uint16_t* weight, int64_t ld_weight,
                      int64_t rows, int64_t H, int64_t V, int64_t v_begin, const float* temp, float temp_scalar,
                      const int64_t* targets, const float* lse, const float* entropy, const float* grad_logprob,
                      const float* grad_entropy, uint16_t* g, int64_t ld_g, int64_t v_pad, uint16_t* gt,
                      int64_t ld_gt, int64_t t_pad, void* stream) {
  // the 64-wide sweep with an even stage count writes G^T and needs it; the other forms never do
  if (v_pad % 64 != 0 || ld_g > kMaxTileLd || (gt != nullptr) != fused_grad_writes_transpose(H, ld_hidden, ld_weight) ||
      (gt && (t_pad % 8 != 0 || t_pad < rows || ld_gt % 8 != 0 || ld_gt < t_pad ||
              (reinterpret_cast<uintptr_t>(gt) & 15) != 0)))
    return int(hipErrorInvalidValue);
  EpiArgs ep{};
  ep.gt = gt;
  ep.ld_gt = ld_gt;
  ep.t_pad = t_pad;
  ep.lse = lse;
  ep.entropy = entropy;
  ep.grad_logprob = grad_logprob;
  ep.grad_entropy = grad_entropy;
  ep.g = g;
  ep.ld_g = ld_g;
  ep.v_begin = v_begin;
  ep.v_pad = v_pad;
  return launch_sweep<kEpiGrad>(hidden, ld_hidden, weight, ld_weight, rows, H, V, temp, temp_scalar, targets,
                                nullptr, nullptr, ep, stream);
}

int launch_fused_logits(const uint16_t* hidden, int64_t ld_hidden, const uint16_t* weight, int64_t ld_weight,
                        int64_t rows, int64_t H, int64_t V, uint16_t* out, int64_t ld_out, void* stream) {
  if (ld_out > kMaxTileLd || ld_out % 4 != 0) return int(hipErrorInvalidValue);
  EpiArgs ep{};
  ep.g = out;
  ep.ld_g = ld_out;
  return launch_sweep<kEpiLogits>(hidden, ld_hidden, weight, ld_weight, rows, H, V, nullptr, 1.0f, nullptr, nullptr,
                                  nullptr, ep, stream);
}

int launch_gemm_nt(const uint16_t* a, int64_t lda, int64_t M, const uint16_t* b, int64_t ldb, int64_t N, int64_t K,
                   float* c, int64_t ldc, bool accumulate, void* stream) {
  EpiArgs ep{};
  ep.c = c;
  ep.ldc = ldc;
  ep.accumulate = accumulate ? 1 : 0;
  // the sweep's "weight" rows are the M axis, its "hidden" rows the N axis
  return launch_sweep<kEpiStore>(b, ldb, a, lda, N, K, M, nullptr, 1.0f, nullptr, nullptr, nullptr, ep, stream);
}

int launch_transpose_pad(const uint16_t* src, int64_t ld_s, int64_t R, int64_t C, uint16_t* dst, int64_t ld_d,
                         int64_t R_pad, void* stream) {
  if (C <= 0 || R_pad <= 0) return 0;
  const int64_t gx = (C + 63) / 64, gy = (R_pad + 63) / 64;
  if (gx > 0x7FFFFFFF || gy > 65535) return int(hipErrorInvalidConfiguration);
  transpose_pad_kernel<<<dim3(unsigned(gx), unsigned(gy)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      src, ld_s, R, C, dst, ld_d, R_pad);
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
