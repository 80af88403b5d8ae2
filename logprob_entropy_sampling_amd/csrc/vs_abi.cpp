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

size_t support_ws_bytes(const vs_source* s) {
  return round_up(size_t(s->T) * 4) + round_up(4) + full_ws_bytes(s, s->T);
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
    default: return "unknown status code";
  }
}

size_t vs_workspace_size(int32_t op, const vs_source* src, int64_t width) {
  (void)width;
  if (!src) return 0;
  switch (op) {
    case VS_OP_SCORE_FULL: return full_ws_bytes(src, src->T);
    case VS_OP_SCORE_SUPPORT: return support_ws_bytes(src);
    case VS_OP_SCORE_TRANSFORMS: return round_up(vs::transforms_workspace_bytes(src->T, src->V));
    case VS_OP_L1_DISTANCE: return round_up(vs::l1_workspace_bytes(src->T, src->V));
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
                                  full_vocab_fallback, logprob, entropy, row_status, fb_list, fb_count, stream);
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
  if (src->kind != VS_SRC_LOGITS || src->logits_dtype != VS_BF16) return VS_E_UNSUPPORTED;
  if (!top_k || !top_p || !min_p || !target_ids || !logprob) return VS_E_NULL;
  if (support_ids_cap < 0 || support_ids_cap > kMaxDim) return VS_E_PARAM;
  if (support_ids_cap == 0) support_ids_out = nullptr;
  if (support_ids_out && support_ids_cap > vs::kTransformsMaxCap) return VS_E_UNSUPPORTED;
  rc = check_workspace(workspace, workspace_bytes, round_up(vs::transforms_workspace_bytes(src->T, src->V)));
  if (rc) return rc;
  vs::timer_mark(0, stream);
  rc = vs::launch_transforms(static_cast<const uint16_t*>(src->logits), src->ld_logits, src->T, src->V,
                             src->temperature, src->temperature_scalar, top_k, top_p, min_p, target_ids, logprob,
                             entropy, row_status, support_len, threshold_logit, threshold_ties, support_ids_out,
                             support_ids_cap, full_lse, static_cast<uint8_t*>(workspace), stream);
  vs::timer_mark(1, stream);
  if (rc == -1) return VS_E_UNSUPPORTED;
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

int vs_sweep_timer(int32_t enable) { return vs::timer_enable(enable != 0) ? VS_E_DEVICE : VS_OK; }

int vs_sweep_timer_ms(float* ms) {
  if (!ms) return VS_E_NULL;
  const int rc = vs::timer_read_ms(ms);
  return rc == 0 ? VS_OK : rc == 2 ? VS_E_PARAM : VS_E_DEVICE;
}

}  // extern "C"
