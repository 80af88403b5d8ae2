// Internal launchers (host side).  Plain C++ types only; every pointer is a
// device pointer, `stream` is a hipStream_t.  Each returns 0 on success or a
// hipError_t value.  Argument validation is done by the C ABI layer before
// any of these is called.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace vs {

// Logits source description shared by the logits-input kernels.
struct LogitsArg {
  const void* ptr;
  int dtype;  // VS_F32 / VS_BF16
  int64_t ld;
};

// Tile widths of the two full-vocabulary sweeps.
constexpr int kFusedTileV = 256;   // vocabulary rows per MFMA tile, fused input
constexpr int kFusedTileT = 256;   // token rows per MFMA tile, fused input

// Full-vocabulary scoring of materialised logits, one workgroup per row slot
// (row_map / row_count nullable); writes the row outputs directly (mode as
// for launch_merge).
int launch_logits_rows(LogitsArg lg, int64_t rows, int64_t V, const float* temp, float temp_scalar,
                       const int32_t* row_map, const int32_t* row_count, const int64_t* targets, float* lse,
                       float* logprob, float* entropy, uint8_t* status, int mode, void* stream);

// bf16 MFMA projection of hidden x weight^T with the per-tile reduction fused
// in; writes partials[slot * n_vtiles + vtile] and zy_raw[slot] (the raw
// logit of the target id).
int launch_fused_partials(const uint16_t* hidden, int64_t ld_hidden, const uint16_t* weight, int64_t ld_weight,
                          int64_t rows, int64_t H, int64_t V, const float* temp, float temp_scalar,
                          const int64_t* targets, const int32_t* row_map, const int32_t* row_count,
                          void* partials, float* zy_raw, void* stream);

// Largest row stride of the bf16 outputs of the sweep (G, the logits block):
// a tile's element offsets stay below 2^31.
constexpr int64_t kMaxTileLd = int64_t(1) << 23;

// The gradient sweep: the same tiles over weight rows [0, V) (vocabulary ids
// v_begin + v) x hidden rows [0, rows); writes the logits' gradient as bf16
// into g [rows][ld_g] (ld_g <= kMaxTileLd), zeros in columns V .. v_pad-1 (v_pad a multiple of 64),
// and, where fused_grad_writes_transpose(H, ld_hidden, ld_weight), its transpose into gt [V][ld_gt],
// zeros in columns rows .. t_pad-1 (t_pad and ld_gt multiples of 8, gt 16-byte
// aligned).  gt must be given exactly where that holds (else an error is returned).
bool fused_grad_writes_transpose(int64_t H, int64_t ld_hidden, int64_t ld_weight);
int launch_fused_grad(const uint16_t* hidden, int64_t ld_hidden, const uint16_t* weight, int64_t ld_weight,
                      int64_t rows, int64_t H, int64_t V, int64_t v_begin, const float* temp, float temp_scalar,
                      const int64_t* targets, const float* lse, const float* entropy, const float* grad_logprob,
                      const float* grad_entropy, uint16_t* g, int64_t ld_g, int64_t v_pad, uint16_t* gt,
                      int64_t ld_gt, int64_t t_pad, void* stream);

// c[m][n] (+)= sum_k a[m][k] b[n][k] (bf16 in, fp32 out; K a multiple of 8,
// lda, ldb multiples of 8, a and b 16-byte aligned): the sweep's MFMA loop
// with a plain store.
int launch_gemm_nt(const uint16_t* a, int64_t lda, int64_t M, const uint16_t* b, int64_t ldb, int64_t N, int64_t K,
                   float* c, int64_t ldc, bool accumulate, void* stream);

// logits [rows][ld_out] (bf16, nearest even) = hidden [rows][H] . weight [V][H]^T:
// the sweep's MFMA loop with a bf16 store (ld_out a multiple of 4, >= V,
// <= kMaxTileLd; else an error is returned).
int launch_fused_logits(const uint16_t* hidden, int64_t ld_hidden, const uint16_t* weight, int64_t ld_weight,
                        int64_t rows, int64_t H, int64_t V, uint16_t* out, int64_t ld_out, void* stream);

// dst[c][r] = src[r][c] (bf16), zeros for R <= r < R_pad.
int launch_transpose_pad(const uint16_t* src, int64_t ld_s, int64_t R, int64_t C, uint16_t* dst, int64_t ld_d,
                         int64_t R_pad, void* stream);

// fp32 -> bf16 (round to nearest even) of hidden rows into a packed [rows, H] buffer.
int launch_round_hidden(const float* hidden, int64_t ld_hidden, int64_t rows, int64_t H, uint16_t* out,
                        void* stream);

// Fixed-order merge of the per-tile partials into the row outputs.
enum MergeMode { kMergeFull = 0, kMergeFallback = 1 };
int launch_merge(const void* partials, int n_tiles, int tiles_per_chunk, int64_t rows, const int32_t* row_map,
                 const int32_t* row_count, const float* temp, float temp_scalar, const int64_t* targets, int64_t V,
                 LogitsArg lg, const float* zy_raw, float* lse, float* logprob, float* entropy, uint8_t* status,
                 int mode, void* stream);

// Recorded support over materialised logits (one wave per row).
int launch_support_logits(LogitsArg lg, int64_t rows, int64_t V, const float* temp, float temp_scalar,
                          const int64_t* ids, int64_t width, int64_t ld_ids, const int64_t* targets,
                          const uint8_t* fallback, float* logprob, float* entropy, uint8_t* status,
                          int32_t* fb_list, int32_t* fb_count, void* stream);

// Recorded support through selected weight rows (gathered projection).
int launch_support_fused(const void* hidden, int hidden_dtype, int64_t ld_hidden, const uint16_t* weight,
                         int64_t ld_weight, int64_t rows, int64_t H, int64_t V, const float* temp,
                         float temp_scalar, const int64_t* ids, int64_t width, int64_t ld_ids,
                         const int64_t* targets, const uint8_t* fallback, float* logprob, float* entropy,
                         uint8_t* status, int32_t* fb_list, int32_t* fb_count, int32_t* order_ws, void* stream);
// The workgroup order of the per-row support kernels on a hidden/weight source
// (rows ranked by their id count, dealt out so each CU gets a near-equal
// share) in ws[0, rows), using ws[rows, 2 rows) for the counts; returns ws, or
// null when there is nothing to balance (width <= 1, fewer than 2 rows per CU).
// A row's results do not depend on the order.
const int32_t* support_row_order(const int64_t* ids, int64_t width, int64_t ld_ids, int64_t rows, int32_t* ws,
                                 void* stream);

// Zero a small int32 buffer with a kernel (not a memset node).
int launch_zero_i32(int32_t* p, int64_t n, void* stream);

// Backward of recorded-support scoring through the projection (bf16 hidden
// [rows][ld_hidden], W [V][ld_weight]): d_hidden [rows][ld_dh] (every row
// written, zeros where no gradient), d_weight [V][ld_dw] (every row written)
// or nullptr.  Workspace: support_backward_workspace_bytes(rows, width, V).
size_t support_backward_workspace_bytes(int64_t rows, int64_t width, int64_t V);
int launch_support_backward(const uint16_t* hidden, int64_t ld_hidden, const uint16_t* weight, int64_t ld_weight,
                            int64_t rows, int64_t H, int64_t V, const float* temp, float temp_scalar,
                            const int64_t* ids, int64_t width, int64_t ld_ids, const int64_t* targets,
                            const float* grad_logprob, const float* grad_entropy, float* d_hidden, int64_t ld_dh,
                            float* d_weight, int64_t ld_dw, void* workspace, void* stream);

// Sampling transforms over bf16 logits (one workgroup per row).  Rows up to
// 20 * 512 * 8 tokens are held in registers; longer ones are counted by one
// kernel and finished by another (several rows per CU), which pass a record
// per row through the workspace (up to 2048 dense ids; more use a one-kernel
// streaming form).  A row that repeats one logit 65536+ times is re-done by a
// 32-bit-count streaming kernel (flagged in `handoff`, the first bytes of the
// workspace).  More than kTransformsMaxCap dense ids: returns -1.  targets may
// be null (every row then scores token 0: the caller wants the support only).
constexpr int64_t kTransformsMaxCap = 4096;  // dense ids are sorted in LDS
size_t transforms_workspace_bytes(int64_t rows, int64_t V);
int launch_transforms(const uint16_t* logits, int64_t ld, int64_t rows, int64_t V, const float* temp,
                      float temp_scalar, const int32_t* top_k, const float* top_p, const float* min_p,
                      const int64_t* targets, float* logprob, float* entropy, uint8_t* status,
                      int32_t* support_len, float* threshold_logit, int32_t* threshold_ties, int64_t* ids_out,
                      int64_t cap, float* full_lse, float* row_max, uint8_t* handoff, void* stream);

// Seeded Gumbel draw over the transforms' support descriptor (status and
// descriptor from launch_transforms, row_max its largest logit per row);
// out_status (nullable) gets the BAD_INPUT bit.  Local row r draws with the
// generator's row word row0 + r.  order (nullable): the local rows in the
// order the workgroups take them (launch_order_rows), which changes no draw.
// ids (nullable): the transforms' dense support ids [rows][cap], cap <= 64,
// with support_len: a row whose whole support is listed is drawn from the list.
int launch_sample(const uint16_t* logits, int64_t ld, int64_t rows, int64_t V, const float* temp, float temp_scalar,
                  const uint8_t* status, const float* threshold_logit, const int32_t* threshold_ties,
                  const float* row_max, uint64_t seed, uint64_t offset, int64_t* sampled, uint8_t* out_status,
                  int64_t row0, const int32_t* order, const int64_t* ids, int64_t cap, const int32_t* support_len,
                  void* stream);
// A permutation of rows [0, rows) into order[rows], the largest supports first
// (support_len and status from launch_transforms): the sampler's row order.
int launch_order_rows(const int32_t* support_len, const uint8_t* status, int64_t rows, int32_t* order, void* stream);

// Draft/target softmax L1.
int launch_l1(LogitsArg target, LogitsArg draft, int64_t rows, int64_t V, float* l1, float* accept,
              void* workspace, void* stream);
size_t l1_workspace_bytes(int64_t rows, int64_t V);

// Number of compute units of the current device (cached per device); 0 or a
// hipError_t value.
int device_cu_count(int* ncu);

// Weighted L1 distillation loss: per-row l1 / accept, loss_out = {num, den,
// num / den}, and (grad non-NULL) the draft-logit gradient [rows, ld_grad] of
// grad_dtype.  Workspace: l1_loss_workspace_bytes(rows).
size_t l1_loss_workspace_bytes(int64_t rows);
int launch_l1_loss(LogitsArg target, LogitsArg draft, int64_t rows, int64_t V, const float* weights,
                   float grad_scale, float* l1, float* accept, float* loss_out, void* grad, int grad_dtype,
                   int64_t ld_grad, void* workspace, void* stream);

// Timing bracket around the sweep kernel(s) of each call (diagnostics).
// timer_enable returns 0 or 1 (event creation failed); timer_read_ms returns
// 0, 1 (HIP error) or 2 (no bracket recorded since enabling).
int timer_enable(int on);
void timer_mark(int stop, void* stream);
int timer_read_ms(float* ms);

}  // namespace vs
