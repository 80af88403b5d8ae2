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
                         uint8_t* status, int32_t* fb_list, int32_t* fb_count, void* stream);

// Zero a small int32 buffer with a kernel (not a memset node).
int launch_zero_i32(int32_t* p, int64_t n, void* stream);

// Sampling transforms over bf16 logits (one workgroup per row).  Rows up to
// 20 * 512 * 8 tokens are held in registers; longer ones are counted by one
// kernel and finished by another (several rows per CU), which pass a record
// per row through the workspace (up to 2048 dense ids; more use a one-kernel
// streaming form).  A row that repeats one logit 65536+ times is re-done by a
// 32-bit-count streaming kernel (flagged in `handoff`, the first bytes of the
// workspace).  More than kTransformsMaxCap dense ids: returns -1.
constexpr int64_t kTransformsMaxCap = 4096;  // dense ids are sorted in LDS
size_t transforms_workspace_bytes(int64_t rows, int64_t V);
int launch_transforms(const uint16_t* logits, int64_t ld, int64_t rows, int64_t V, const float* temp,
                      float temp_scalar, const int32_t* top_k, const float* top_p, const float* min_p,
                      const int64_t* targets, float* logprob, float* entropy, uint8_t* status,
                      int32_t* support_len, float* threshold_logit, int32_t* threshold_ties, int64_t* ids_out,
                      int64_t cap, float* full_lse, uint8_t* handoff, void* stream);

// Draft/target softmax L1.
int launch_l1(LogitsArg target, LogitsArg draft, int64_t rows, int64_t V, float* l1, float* accept,
              void* workspace, void* stream);
size_t l1_workspace_bytes(int64_t rows, int64_t V);

// Timing bracket around the sweep kernel(s) of each call (diagnostics).
// timer_enable returns 0 or 1 (event creation failed); timer_read_ms returns
// 0, 1 (HIP error) or 2 (no bracket recorded since enabling).
int timer_enable(int on);
void timer_mark(int stop, void* stream);
int timer_read_ms(float* ms);

}  // namespace vs
