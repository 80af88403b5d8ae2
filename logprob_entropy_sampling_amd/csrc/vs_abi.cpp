// C ABI of libvocabscore.so: argument validation, workspace layout, launches.
//
// This translation unit includes no HIP header: every check below runs on
// the host before anything is enqueued, and a failed check returns its
// VS_E_* code without touching the device (one place, one early error,
// never a silent fallback - xorl issue #71, "Proposed direction" item 5).
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/vocabscore.h"
#include "launch.h"

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxH = int64_t(1) << 24;
constexpr int64_t kMaxSupportH = 16384;  // hidden row staged in LDS by the support kernel
constexpr int64_t kMaxWidth = 1024;
constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t esize(int dt) { return dt == VS_BF16 ? 2 : 4; }
bool dtype_ok(int dt) { return dt == VS_BF16 || dt == VS_F32; }

// Sequential carving of the caller's workspace.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  void* take(size_t bytes) {
    void* r = base ? base + off : nullptr;
    off += round_up(bytes);
    return r;
  }
};

int64_t n_fused_tiles(int64_t V) { return (V + vs::kFusedTileV - 1) / vs::kFusedTileV; }

int check_source(const vs_source* s) {
  if (!s) return VS_E_NULL;
  if (s->T < 1 || s->T > kMaxDim || s->V < 1 || s->V > kMaxDim) return VS_E_SHAPE;
  if (!s->temperature && !(std::isfinite(s->temperature_scalar) && s->temperature_scalar > 0.0f)) return VS_E_PARAM;
  if (s->kind == VS_SRC_LOGITS) {
    if (!s->logits) return VS_E_NULL;
    if (!dtype_ok(s->logits_dtype)) return VS_E_DTYPE;
    if (s->ld_logits < s->V) return VS_E_SHAPE;
    if (!aligned(s->logits, esize(s->logits_dtype))) return VS_E_ALIGN;
    return VS_OK;
  }
  if (s->kind == VS_SRC_HIDDEN_WEIGHT) {
    if (!s->hidden || !s->weight) return VS_E_NULL;
    if (s->weight_dtype != VS_BF16 || !dtype_ok(s->hidden_dtype)) return VS_E_DTYPE;
    if (s->H < 8 || s->H >= kMaxH || s->H % 8 != 0) return VS_E_SHAPE;
    if (s->ld_hidden < s->H || s->ld_weight < s->H) return VS_E_SHAPE;
    if (s->ld_hidden % 8 != 0 || s->ld_weight % 8 != 0) return VS_E_ALIGN;
    if (!aligned(s->hidden, 16) || !aligned(s->weight, 16)) return VS_E_ALIGN;
    return VS_OK;
  }
  return VS_E_PARAM;
}

int check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return VS_OK;
  if (!ws || !aligned(ws, kAlign) || have < need) return VS_E_WORKSPACE;
  return VS_OK;
}

// Workspace of a full-vocabulary sweep over `rows` rows (also the fallback's).
struct FullWs {
  void* partials = nullptr;
  float* zy = nullptr;
  uint16_t* hidden_bf16 = nullptr;
};

size_t full_ws_bytes(const vs_source* s, int64_t rows) {
  if (s->kind == VS_SRC_LOGITS) return 0;  // the row kernel needs no workspace
  size_t b = round_up(size_t(rows) * size_t(n_fused_tiles(s->V)) * 16) + round_up(size_t(rows) * 4);
  if (s->hidden_dtype == VS_F32) b += round_up(size_t(s->T) * size_t(s->H) * 2);
  return b;
}

FullWs carve_full(Carver& c, const vs_source* s, int64_t rows) {
  FullWs w;
  if (s->kind == VS_SRC_LOGITS) return w;
  w.partials = c.take(size_t(rows) * size_t(n_fused_tiles(s->V)) * 16);
  w.zy = static_cast<float*>(c.take(size_t(rows) * 4));
  if (s->hidden_dtype == VS_F32) w.hidden_bf16 = static_cast<uint16_t*>(c.take(size_t(s->T) * size_t(s->H) * 2));
  return w;
}

// Transforms over a hidden/weight source: the sweep writes the bf16 logits of
// blocks of up to kXfRows token rows into the workspace ([rows][ld], ld = V
// rounded up to 8 so that every row is 16-byte aligned), and the transforms
// (and the sampler) run on each block before the next is written.  An fp32
// hidden state is rounded to bf16 first.
constexpr int64_t kXfRows = 2048;
struct XfDims {
  int64_t rows, ld;
};
XfDims xf_dims(const vs_source* s) {
  return XfDims{s->T < kXfRows ? s->T : kXfRows, (s->V + 7) / 8 * 8};
}
// the transforms' workspace, plus (hidden/weight source) the logits block and
// the rounded hidden state
size_t xf_ws_bytes(const vs_source* s) {
  if (s->kind != VS_SRC_HIDDEN_WEIGHT) return round_up(vs::transforms_workspace_bytes(s->T, s->V));
  const XfDims d = xf_dims(s);
  size_t b = round_up(size_t(d.rows) * size_t(d.ld) * 2) + round_up(vs::transforms_workspace_bytes(d.rows, s->V));
  if (s->hidden_dtype == VS_F32) b += round_up(size_t(s->T) * size_t(s->H) * 2);
  return b;
}

// the sampler: logprob, status, row maxima, threshold logit, ties and support
// lengths (when the caller passes none), the rows' draw order, the dense ids
// of supports of up to kSampleIdsCap tokens, then the transforms' own workspace
constexpr int64_t kSampleIdsCap = 64;
size_t sample_ws_bytes(const vs_source* s) {
  const size_t T = size_t(s->T);
  return round_up(T * 4) + round_up(T) + 5 * round_up(T * 4) + round_up(T * kSampleIdsCap * 8) + xf_ws_bytes(s);
}

template <class P>
P* at_row(P* p, int64_t row, int64_t stride = 1) {
  return p ? p + row * stride : nullptr;
}

// The logits blocks of a hidden/weight source, one after the other: for each
// block, fn(logits, ld, first row, rows, transforms workspace) runs after the
// block's sweep.  Returns a VS_ status.
template <class Fn>
int over_logit_blocks(const vs_source* src, Carver& c, void* stream, Fn fn) {
  const XfDims d = xf_dims(src);
  const uint16_t* hid = static_cast<const uint16_t*>(src->hidden);
  int64_t ldh = src->ld_hidden;
  if (src->hidden_dtype == VS_F32) {
    uint16_t* hb = static_cast<uint16_t*>(c.take(size_t(src->T) * size_t(src->H) * 2));
    if (vs::launch_round_hidden(static_cast<const float*>(src->hidden), src->ld_hidden, src->T, src->H, hb, stream))
      return VS_E_DEVICE;
    hid = hb;
    ldh = src->H;
  }
  uint16_t* L = static_cast<uint16_t*>(c.take(size_t(d.rows) * size_t(d.ld) * 2));
  uint8_t* tws = static_cast<uint8_t*>(c.take(vs::transforms_workspace_bytes(d.rows, src->V)));
  for (int64_t r0 = 0; r0 < src->T; r0 += d.rows) {
    const int64_t n = src->T - r0 < d.rows ? src->T - r0 : d.rows;
    if (vs::launch_fused_logits(hid + r0 * ldh, ldh, static_cast<const uint16_t*>(src->weight), src->ld_weight, n,
                                src->H, src->V, L, d.ld, stream))
      return VS_E_DEVICE;
    const int rc = fn(static_cast<const uint16_t*>(L), d.ld, r0, n, tws);
    if (rc) return rc;
  }
  return VS_OK;
}

// Backward of full-vocabulary scoring through the fused projection: per
// vocabulary chunk of Vc rows (a multiple of the 256-row tile), the logits'
// gradient G [T][Vc] and G^T [Vc][Tp] (bf16), W^T of the chunk [H][Vc], and
// once the hidden state's transpose [H][Tp] (Tp = T rounded up to 64, the
// GEMMs' K multiple) and, for an fp32 hidden state, its bf16 copy.
struct BwdDims {
  int64_t vc, tp;
};
BwdDims bwd_dims(const vs_source* s, int64_t vocab_chunk) {
  const int64_t tile = vs::kFusedTileV;
  int64_t vc = vocab_chunk < tile ? tile : (vocab_chunk + tile - 1) / tile * tile;
  const int64_t vmax = (s->V + tile - 1) / tile * tile;
  if (vc > vmax) vc = vmax;
  if (vc > vs::kMaxTileLd) vc = vs::kMaxTileLd;  // G's row stride (a multiple of the tile)
  return BwdDims{vc, (s->T + 63) / 64 * 64};
}
size_t backward_ws_bytes(const vs_source* s, int64_t vocab_chunk) {
  if (s->kind != VS_SRC_HIDDEN_WEIGHT) return 0;
  const BwdDims d = bwd_dims(s, vocab_chunk);
  const size_t T = size_t(s->T), H = size_t(s->H);
  size_t b = 0;
  if (s->hidden_dtype == VS_F32) b += round_up(T * H * 2);
  b += round_up(H * size_t(d.tp) * 2);         // hidden^T
  b += round_up(T * size_t(d.vc) * 2);         // G
  b += round_up(size_t(d.vc) * size_t(d.tp) * 2);  // G^T
  b += round_up(H * size_t(d.vc) * 2);         // W^T of a chunk
  return b;
}

// the backward of recorded-support scoring: the bf16 copy of an fp32 hidden
// state, then the kernels' own arrays (dX per pair, row flags, per-id counts,
// offsets and fill, the pair list)
size_t support_bwd_ws_bytes(const vs_source* s, int64_t width) {
  if (s->kind != VS_SRC_HIDDEN_WEIGHT) return 0;
  size_t b = round_up(vs::support_backward_workspace_bytes(s->T, width, s->V));
  if (s->hidden_dtype == VS_F32) b += round_up(size_t(s->T) * size_t(s->H) * 2);
  return b;
}

size_t support_ws_bytes(const vs_source* s) {
  return round_up(size_t(s->T) * 4) + round_up(4) + 2 * round_up(size_t(s->T) * 4) + full_ws_bytes(s, s->T);
}

// Full-vocabulary sweep + merge over `rows` slots (row_map/row_count nullable).
int run_full(const vs_source* s, const FullWs& w, int64_t rows, const int32_t* row_map, const int32_t* row_count,
             const int64_t* targets, int64_t vocab_chunk, float* lse, float* logprob, float* entropy,
             uint8_t* status, int mode, bool timed, void* stream) {
  vs::LogitsArg lg{s->logits, s->logits_dtype, s->ld_logits};
  int rc;
  if (s->kind == VS_SRC_LOGITS) {  // one pass, one kernel, no partials
    (void)w;
    (void)vocab_chunk;
    if (timed) vs::timer_mark(0, stream);
    rc = vs::launch_logits_rows(lg, rows, s->V, s->temperature, s->temperature_scalar, row_map, row_count, targets,
                                lse, logprob, entropy, status, mode, stream);
    if (timed) vs::timer_mark(1, stream);
    return rc ? VS_E_DEVICE : VS_OK;
  }
  const uint16_t* hid = static_cast<const uint16_t*>(s->hidden);
  int64_t ldh = s->ld_hidden;
  if (s->hidden_dtype == VS_F32) {
    rc = vs::launch_round_hidden(static_cast<const float*>(s->hidden), s->ld_hidden, s->T, s->H, w.hidden_bf16,
                                 stream);
    if (rc) return VS_E_DEVICE;
    hid = w.hidden_bf16;
    ldh = s->H;
  }
  const int64_t nt = n_fused_tiles(s->V);
  int64_t tpc = vocab_chunk / vs::kFusedTileV;
  if (tpc < 1) tpc = 1;
  if (timed) vs::timer_mark(0, stream);
  rc = vs::launch_fused_partials(hid, ldh, static_cast<const uint16_t*>(s->weight), s->ld_weight, rows, s->H, s->V,
                                 s->temperature, s->temperature_scalar, targets, row_map, row_count, w.partials,
                                 w.zy, stream);
  if (timed) vs::timer_mark(1, stream);
  if (rc) return VS_E_DEVICE;
  rc = vs::launch_merge(w.partials, int(nt), int(tpc), rows, row_map, row_count, s->temperature,
                        s->temperature_scalar, targets, s->V, lg, w.zy, lse, logprob, entropy, status, mode, stream);
  return rc ? VS_E_DEVICE : VS_OK;
}

}  // namespace

extern "C" {

int32_t vs_version(void) { return 10000; }

const char* vs_status_string(int32_t code) {
  switch (code) {
    case VS_OK: return "ok";
    case VS_E_NULL: return "a required pointer is NULL";
    case VS_E_SHAPE: return "a size is out of range or a leading dimension is too small";
    case VS_E_DTYPE: return "unsupported dtype or dtype combination";
    case VS_E_ALIGN: return "a pointer or leading dimension breaks an alignment rule";
    case VS_E_PARAM: return "a scalar parameter is out of range";
    case VS_E_WORKSPACE: return "workspace is NULL, not 256-byte aligned, or smaller than vs_workspace_size()";
    case VS_E_UNSUPPORTED: return "this request is valid but not implemented for this source kind";
    case VS_E_DEVICE: return "a HIP kernel launch failed";
    case VS_E_SCRATCH: return "the call needs more scratch than vs_score_full_noalloc holds (vs_noalloc_scratch_bytes)";
    default: return "unknown status code";
  }
}

size_t vs_workspace_size(int32_t op, const vs_source* src, int64_t width) {
  if (!src) return 0;
  switch (op) {
    case VS_OP_SCORE_FULL: return full_ws_bytes(src, src->T);
    case VS_OP_SCORE_SUPPORT: return support_ws_bytes(src);
    case VS_OP_SCORE_TRANSFORMS: return xf_ws_bytes(src);
    case VS_OP_L1_DISTANCE: return round_up(vs::l1_workspace_bytes(src->T, src->V));
    case VS_OP_SAMPLE_TRANSFORMS: return sample_ws_bytes(src);
    case VS_OP_L1_LOSS: return round_up(vs::l1_loss_workspace_bytes(src->T));
    case VS_OP_SCORE_FULL_BACKWARD: return backward_ws_bytes(src, width);
    case VS_OP_SCORE_SUPPORT_BACKWARD: return support_bwd_ws_bytes(src, width);
    default: return 0;
  }
}

int vs_score_full(const vs_source* src, const int64_t* target_ids, int64_t vocab_chunk, float* lse, float* logprob,
                  float* entropy, uint8_t* row_status, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_source(src);
  if (rc) return rc;
  if (!target_ids || !logprob) return VS_E_NULL;
  if (vocab_chunk < 1) return VS_E_PARAM;
  rc = check_workspace(workspace, workspace_bytes, full_ws_bytes(src, src->T));
  if (rc) return rc;
  Carver c(workspace);
  FullWs w = carve_full(c, src, src->T);
  return run_full(src, w, src->T, nullptr, nullptr, target_ids, vocab_chunk, lse, logprob, entropy, row_status,
                  vs::kMergeFull, true, stream);
}

int vs_score_support_ids(const vs_source* src, const int64_t* support_ids, int64_t width, int64_t ld_ids,
                         const int64_t* target_ids, const uint8_t* full_vocab_fallback, int64_t vocab_chunk,
                         float* logprob, float* entropy, uint8_t* row_status, void* workspace,
                         size_t workspace_bytes, void* stream) {
  int rc = check_source(src);
  if (rc) return rc;
  if (!target_ids || !logprob) return VS_E_NULL;
  if (width < 0 || width > kMaxWidth || ld_ids < width) return VS_E_SHAPE;
  if (width > 0 && !support_ids) return VS_E_NULL;
  if (vocab_chunk < 1) return VS_E_PARAM;
  if (src->kind == VS_SRC_HIDDEN_WEIGHT && src->H > kMaxSupportH) return VS_E_UNSUPPORTED;
  rc = check_workspace(workspace, workspace_bytes, support_ws_bytes(src));
  if (rc) return rc;
  Carver c(workspace);
  int32_t* fb_list = static_cast<int32_t*>(c.take(size_t(src->T) * 4));
  int32_t* fb_count = static_cast<int32_t*>(c.take(4));
  int32_t* order_ws = static_cast<int32_t*>(c.take(size_t(src->T) * 8));  // row order, then id counts
  FullWs w = carve_full(c, src, src->T);
  if (full_vocab_fallback && vs::launch_zero_i32(fb_count, 1, stream)) return VS_E_DEVICE;
  vs::timer_mark(0, stream);
  if (src->kind == VS_SRC_LOGITS) {
    vs::LogitsArg lg{src->logits, src->logits_dtype, src->ld_logits};
    rc = vs::launch_support_logits(lg, src->T, src->V, src->temperature, src->temperature_scalar, support_ids,
                                   width, ld_ids, target_ids, full_vocab_fallback, logprob, entropy, row_status,
                                   fb_list, fb_count, stream);
  } else {
    rc = vs::launch_support_fused(src->hidden, src->hidden_dtype, src->ld_hidden,
                                  static_cast<const uint16_t*>(src->weight), src->ld_weight, src->T, src->H, src->V,
                                  src->temperature, src->temperature_scalar, support_ids, width, ld_ids, target_ids,
                                  full_vocab_fallback, logprob, entropy, row_status, fb_list, fb_count, order_ws,
                                  stream);
  }
  vs::timer_mark(1, stream);
  if (rc) return VS_E_DEVICE;
  if (!full_vocab_fallback) return VS_OK;
  // synthetic-EOS rows: full-vocabulary logprob of the listed rows
  return run_full(src, w, src->T, fb_list, fb_count, target_ids, vocab_chunk, nullptr, logprob, entropy,
                  row_status, vs::kMergeFallback, false, stream);
}

int vs_score_transforms(const vs_source* src, const int32_t* top_k, const float* top_p, const float* min_p,
                        const int64_t* target_ids, float* logprob, float* entropy, uint8_t* row_status,
                        int32_t* support_len, float* threshold_logit, int32_t* threshold_ties,
                        int64_t* support_ids_out, int64_t support_ids_cap, float* full_lse, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int rc = check_source(src);
  if (rc) return rc;
  if (src->kind == VS_SRC_LOGITS && src->logits_dtype != VS_BF16) return VS_E_UNSUPPORTED;
  if (src->kind == VS_SRC_HIDDEN_WEIGHT && xf_dims(src).ld > vs::kMaxTileLd) return VS_E_UNSUPPORTED;
  if (!top_k || !top_p || !min_p || !target_ids || !logprob) return VS_E_NULL;
  if (support_ids_cap < 0 || support_ids_cap > kMaxDim) return VS_E_PARAM;
  if (support_ids_cap == 0) support_ids_out = nullptr;
  if (support_ids_out && support_ids_cap > vs::kTransformsMaxCap) return VS_E_UNSUPPORTED;
  rc = check_workspace(workspace, workspace_bytes, xf_ws_bytes(src));
  if (rc) return rc;
  const float* temp = src->temperature;
  // rows [r0, r0 + n) of the program over logits [n][ld]
  auto run = [&](const uint16_t* lg, int64_t ld, int64_t r0, int64_t n, uint8_t* tws) -> int {
    const int r = vs::launch_transforms(lg, ld, n, src->V, at_row(temp, r0), src->temperature_scalar, top_k + r0,
                                        top_p + r0, min_p + r0, target_ids + r0, logprob + r0, at_row(entropy, r0),
                                        at_row(row_status, r0), at_row(support_len, r0), at_row(threshold_logit, r0),
                                        at_row(threshold_ties, r0), at_row(support_ids_out, r0, support_ids_cap),
                                        support_ids_cap, at_row(full_lse, r0), nullptr, tws, stream);
    return r == -1 ? VS_E_UNSUPPORTED : r ? VS_E_DEVICE : VS_OK;
  };
  vs::timer_mark(0, stream);
  if (src->kind == VS_SRC_LOGITS) {
    rc = run(static_cast<const uint16_t*>(src->logits), src->ld_logits, 0, src->T, static_cast<uint8_t*>(workspace));
  } else {
    Carver c(workspace);
    rc = over_logit_blocks(src, c, stream, run);
  }
  vs::timer_mark(1, stream);
  return rc;
}

int vs_sample_transforms(const vs_source* src, const int32_t* top_k, const float* top_p, const float* min_p,
                         uint64_t seed, uint64_t offset, int64_t* sampled_ids, uint8_t* row_status,
                         int32_t* support_len, float* threshold_logit, int32_t* threshold_ties, void* workspace,
                         size_t workspace_bytes, void* stream) {
  int rc = check_source(src);
  if (rc) return rc;
  if (src->kind == VS_SRC_LOGITS && src->logits_dtype != VS_BF16) return VS_E_UNSUPPORTED;
  if (src->kind == VS_SRC_HIDDEN_WEIGHT && xf_dims(src).ld > vs::kMaxTileLd) return VS_E_UNSUPPORTED;
  if (!top_k || !top_p || !min_p || !sampled_ids) return VS_E_NULL;
  rc = check_workspace(workspace, workspace_bytes, sample_ws_bytes(src));
  if (rc) return rc;
  const int64_t T = src->T;
  Carver c(workspace);
  float* lp = static_cast<float*>(c.take(size_t(T) * 4));
  uint8_t* st = static_cast<uint8_t*>(c.take(size_t(T)));
  float* row_max = static_cast<float*>(c.take(size_t(T) * 4));
  float* thr = threshold_logit ? threshold_logit : static_cast<float*>(c.take(size_t(T) * 4));
  int32_t* ties = threshold_ties ? threshold_ties : static_cast<int32_t*>(c.take(size_t(T) * 4));
  int32_t* slen = support_len ? support_len : static_cast<int32_t*>(c.take(size_t(T) * 4));
  int32_t* order = static_cast<int32_t*>(c.take(size_t(T) * 4));
  int64_t* ids = static_cast<int64_t*>(c.take(size_t(T) * kSampleIdsCap * 8));
  const float* temp = src->temperature;
  // rows [r0, r0 + n): the support descriptor, then the draw from it
  auto run = [&](const uint16_t* lg, int64_t ld, int64_t r0, int64_t n, uint8_t* tws) -> int {
    int r = vs::launch_transforms(lg, ld, n, src->V, at_row(temp, r0), src->temperature_scalar, top_k + r0,
                                  top_p + r0, min_p + r0, nullptr, lp + r0, nullptr, st + r0, slen + r0,
                                  thr + r0, ties + r0, ids + r0 * kSampleIdsCap, kSampleIdsCap, nullptr,
                                  row_max + r0, tws, stream);
    if (r) return r == -1 ? VS_E_UNSUPPORTED : VS_E_DEVICE;
    // the block's rows, the largest supports first (the draws do not depend on it)
    if (vs::launch_order_rows(slen + r0, st + r0, n, order, stream)) return VS_E_DEVICE;
    r = vs::launch_sample(lg, ld, n, src->V, at_row(temp, r0), src->temperature_scalar, st + r0, thr + r0, ties + r0,
                          row_max + r0, seed, offset, sampled_ids + r0, at_row(row_status, r0), r0, order,
                          ids + r0 * kSampleIdsCap, kSampleIdsCap, slen + r0, stream);
    return r ? VS_E_DEVICE : VS_OK;
  };
  vs::timer_mark(0, stream);
  if (src->kind == VS_SRC_LOGITS) {
    rc = run(static_cast<const uint16_t*>(src->logits), src->ld_logits, 0, T,
             static_cast<uint8_t*>(c.take(vs::transforms_workspace_bytes(T, src->V))));
  } else {
    rc = over_logit_blocks(src, c, stream, run);
  }
  vs::timer_mark(1, stream);
  return rc;
}

int vs_score_full_backward(const vs_source* src, const int64_t* target_ids, const float* lse, const float* entropy,
                           const float* grad_logprob, const float* grad_entropy, int64_t vocab_chunk,
                           float* grad_hidden, int64_t ld_grad_hidden, float* grad_weight, int64_t ld_grad_weight,
                           void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_source(src);
  if (rc) return rc;
  if (src->kind != VS_SRC_HIDDEN_WEIGHT) return VS_E_UNSUPPORTED;
  if (!target_ids || !lse || (grad_entropy && !entropy)) return VS_E_NULL;
  if (!grad_hidden && !grad_weight) return VS_E_NULL;
  if (vocab_chunk < 1) return VS_E_PARAM;
  if ((grad_hidden && ld_grad_hidden < src->H) || (grad_weight && ld_grad_weight < src->H)) return VS_E_SHAPE;
  if (!aligned(grad_hidden, 4) || !aligned(grad_weight, 4)) return VS_E_ALIGN;
  rc = check_workspace(workspace, workspace_bytes, backward_ws_bytes(src, vocab_chunk));
  if (rc) return rc;
  const int64_t T = src->T, H = src->H, V = src->V;
  const BwdDims dm = bwd_dims(src, vocab_chunk);
  Carver c(workspace);
  const uint16_t* hid = static_cast<const uint16_t*>(src->hidden);
  int64_t ldh = src->ld_hidden;
  if (src->hidden_dtype == VS_F32) {
    uint16_t* hb = static_cast<uint16_t*>(c.take(size_t(T) * size_t(H) * 2));
    if (vs::launch_round_hidden(static_cast<const float*>(src->hidden), src->ld_hidden, T, H, hb, stream))
      return VS_E_DEVICE;
    hid = hb;
    ldh = H;
  }
  uint16_t* hT = static_cast<uint16_t*>(c.take(size_t(H) * size_t(dm.tp) * 2));
  uint16_t* G = static_cast<uint16_t*>(c.take(size_t(T) * size_t(dm.vc) * 2));
  uint16_t* GT = static_cast<uint16_t*>(c.take(size_t(dm.vc) * size_t(dm.tp) * 2));
  uint16_t* WT = static_cast<uint16_t*>(c.take(size_t(H) * size_t(dm.vc) * 2));
  const uint16_t* W = static_cast<const uint16_t*>(src->weight);
  if (grad_weight && vs::launch_transpose_pad(hid, ldh, T, H, hT, dm.tp, dm.tp, stream)) return VS_E_DEVICE;
  vs::timer_mark(0, stream);
  for (int64_t v0 = 0; v0 < V; v0 += dm.vc) {
    const int64_t vn = V - v0 < dm.vc ? V - v0 : dm.vc;
    const int64_t vp = (vn + 63) / 64 * 64;
    // G^T comes from the sweep itself where it can write it, else from a transpose of G
    const bool gt_direct = vs::fused_grad_writes_transpose(H, ldh, src->ld_weight);
    if (vs::launch_fused_grad(hid, ldh, W + v0 * src->ld_weight, src->ld_weight, T, H, vn, v0, src->temperature,
                              src->temperature_scalar, target_ids, lse, entropy, grad_logprob, grad_entropy, G, dm.vc,
                              vp, gt_direct ? GT : nullptr, dm.tp, dm.tp, stream))
      return VS_E_DEVICE;
    if (grad_hidden) {  // d_hidden [T][H] (+)= G [T][vp] . (W^T [H][vp])^T
      if (vs::launch_transpose_pad(W + v0 * src->ld_weight, src->ld_weight, vn, H, WT, dm.vc, vp, stream) ||
          vs::launch_gemm_nt(G, dm.vc, T, WT, dm.vc, H, vp, grad_hidden, ld_grad_hidden, v0 > 0, stream))
        return VS_E_DEVICE;
    }
    if (grad_weight) {  // d_weight [vn][H] = G^T [vn][Tp] . (hidden^T [H][Tp])^T
      if ((!gt_direct && vs::launch_transpose_pad(G, dm.vc, T, vn, GT, dm.tp, dm.tp, stream)) ||
          vs::launch_gemm_nt(GT, dm.tp, vn, hT, dm.tp, H, dm.tp, grad_weight + v0 * ld_grad_weight, ld_grad_weight,
                             false, stream))
        return VS_E_DEVICE;
    }
  }
  vs::timer_mark(1, stream);
  return VS_OK;
}

int vs_score_support_backward(const vs_source* src, const int64_t* support_ids, int64_t width, int64_t ld_ids,
                              const int64_t* target_ids, const float* grad_logprob, const float* grad_entropy,
                              float* grad_hidden, int64_t ld_grad_hidden, float* grad_weight, int64_t ld_grad_weight,
                              void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_source(src);
  if (rc) return rc;
  if (src->kind != VS_SRC_HIDDEN_WEIGHT) return VS_E_UNSUPPORTED;
  if ((!support_ids && width > 0) || !target_ids) return VS_E_NULL;
  if (!grad_hidden && !grad_weight) return VS_E_NULL;
  if (width < 0 || width > kMaxWidth || ld_ids < width) return VS_E_SHAPE;
  if (src->T * width > 0x7FFFFFFF) return VS_E_SHAPE;
  if (src->H > kMaxSupportH) return VS_E_UNSUPPORTED;
  if ((grad_hidden && ld_grad_hidden < src->H) || (grad_weight && ld_grad_weight < src->H)) return VS_E_SHAPE;
  if (!aligned(grad_hidden, 4) || !aligned(grad_weight, 4)) return VS_E_ALIGN;
  rc = check_workspace(workspace, workspace_bytes, support_bwd_ws_bytes(src, width));
  if (rc) return rc;
  Carver c(workspace);
  const uint16_t* hid = static_cast<const uint16_t*>(src->hidden);
  int64_t ldh = src->ld_hidden;
  if (src->hidden_dtype == VS_F32) {
    uint16_t* hb = static_cast<uint16_t*>(c.take(size_t(src->T) * size_t(src->H) * 2));
    if (vs::launch_round_hidden(static_cast<const float*>(src->hidden), src->ld_hidden, src->T, src->H, hb, stream))
      return VS_E_DEVICE;
    hid = hb;
    ldh = src->H;
  }
  void* ws = c.take(vs::support_backward_workspace_bytes(src->T, width, src->V));
  vs::timer_mark(0, stream);
  rc = vs::launch_support_backward(hid, ldh, static_cast<const uint16_t*>(src->weight), src->ld_weight, src->T, src->H,
                                   src->V, src->temperature, src->temperature_scalar, support_ids, width, ld_ids,
                                   target_ids, grad_logprob, grad_entropy, grad_hidden, ld_grad_hidden, grad_weight,
                                   ld_grad_weight, ws, stream);
  vs::timer_mark(1, stream);
  return rc ? VS_E_DEVICE : VS_OK;
}

int vs_l1_distance(const void* target_logits, const void* draft_logits, int32_t dtype, int64_t T, int64_t V,
                   int64_t ld_target, int64_t ld_draft, float* l1, float* accept_rate, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!target_logits || !draft_logits || !l1) return VS_E_NULL;
  if (!dtype_ok(dtype)) return VS_E_DTYPE;
  if (T < 1 || T > kMaxDim || V < 1 || V > kMaxDim || ld_target < V || ld_draft < V) return VS_E_SHAPE;
  if (!aligned(target_logits, esize(dtype)) || !aligned(draft_logits, esize(dtype))) return VS_E_ALIGN;
  int rc = check_workspace(workspace, workspace_bytes, round_up(vs::l1_workspace_bytes(T, V)));
  if (rc) return rc;
  vs::timer_mark(0, stream);
  rc = vs::launch_l1(vs::LogitsArg{target_logits, dtype, ld_target}, vs::LogitsArg{draft_logits, dtype, ld_draft}, T,
                     V, l1, accept_rate, workspace, stream);
  vs::timer_mark(1, stream);
  if (rc == -1) return VS_E_UNSUPPORTED;
  return rc ? VS_E_DEVICE : VS_OK;
}

int vs_l1_loss(const void* target_logits, const void* draft_logits, int32_t dtype, int64_t T, int64_t V,
               int64_t ld_target, int64_t ld_draft, const float* weights, float grad_scale, float* l1,
               float* accept_rate, float* loss, void* grad_draft, int32_t grad_dtype, int64_t ld_grad,
               void* workspace, size_t workspace_bytes, void* stream) {
  if (!target_logits || !draft_logits || !l1 || !loss) return VS_E_NULL;
  if (!dtype_ok(dtype) || (grad_draft && !dtype_ok(grad_dtype))) return VS_E_DTYPE;
  if (T < 1 || T > kMaxDim || V < 1 || V > kMaxDim || ld_target < V || ld_draft < V) return VS_E_SHAPE;
  if (grad_draft && ld_grad < V) return VS_E_SHAPE;
  if (!aligned(target_logits, esize(dtype)) || !aligned(draft_logits, esize(dtype))) return VS_E_ALIGN;
  if (grad_draft && !aligned(grad_draft, esize(grad_dtype))) return VS_E_ALIGN;
  if (!std::isfinite(grad_scale)) return VS_E_PARAM;
  int rc = check_workspace(workspace, workspace_bytes, round_up(vs::l1_loss_workspace_bytes(T)));
  if (rc) return rc;
  vs::timer_mark(0, stream);
  rc = vs::launch_l1_loss(vs::LogitsArg{target_logits, dtype, ld_target}, vs::LogitsArg{draft_logits, dtype, ld_draft},
                          T, V, weights, grad_scale, l1, accept_rate, loss, grad_draft, grad_dtype, ld_grad, workspace,
                          stream);
  vs::timer_mark(1, stream);
  return rc ? VS_E_DEVICE : VS_OK;
}

int vs_sweep_timer(int32_t enable) { return vs::timer_enable(enable != 0) ? VS_E_DEVICE : VS_OK; }

int vs_sweep_timer_ms(float* ms) {
  if (!ms) return VS_E_NULL;
  const int rc = vs::timer_read_ms(ms);
  return rc == 0 ? VS_OK : rc == 2 ? VS_E_PARAM : VS_E_DEVICE;
}

}  // extern "C"
