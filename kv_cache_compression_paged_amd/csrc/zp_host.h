// Internal host helpers shared by the library's C++ files: thread-local error
// messages and the launchers each kernel file exports.
#pragma once

#include <cstddef>
#include <cstdint>

#include "zipage.h"

namespace zp {

// Stores a printf-style message as this thread's last error.
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
// set_error + return code.
zp_status fail(zp_status code, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));

// Geometry every kernel of one compression call shares (all sizes checked).
struct CompressGeom {
  int32_t R, L, Hkv, Hq, G, d, b, n_max, k, w, wG, n_cap, num_blocks;
  int32_t max_blocks, num_slots;
  int32_t dtype, q_dtype;
  uint32_t flags;
  float w_attn, w_global, w_red, scale_log2;
};

// Launchers (defined next to their kernels). Each returns ZP_OK or ZP_EHIP
// (launch error), after recording the error text.
zp_status launch_compress(const CompressGeom& g, const zp_kv_pool& pool,
                          const zp_batch& batch, const void* q_window,
                          float* global_scores,
                          const zp_compress_out& out, int32_t* err, void* stream);
// Split-unit schedule (compress_split.hip): workspace size, whether a call
// can use it, and its launcher (the workspace holds the error word first).
size_t split_workspace_bytes();
bool split_eligible(const CompressGeom& g, size_t workspace_bytes);
zp_status launch_compress_split(const CompressGeom& g, const zp_kv_pool& pool,
                                const zp_batch& batch, const void* q_window,
                                float* global_scores, const zp_compress_out& out,
                                void* workspace, void* stream);
zp_status launch_global(const CompressGeom& g, float* global_scores,
                        const zp_batch& batch, const int32_t* keep,
                        const float* attn, void* stream);

zp_status launch_redundancy_full(const CompressGeom& g, const zp_kv_pool& pool,
                                 const zp_batch& batch, float* red_block, float* red_all,
                                 int32_t* err, void* stream);
zp_status launch_capture(void* q_window, const void* q, const int32_t* slot,
                         const int32_t* pos, int32_t num_reqs, int32_t layers,
                         int32_t num_slots, int32_t window, int32_t row_bytes,
                         void* stream);

struct DecodeGeom {
  int32_t R, L, Hkv, Hq, G, d, b, num_blocks, max_blocks, dtype, q_dtype, splits;
  float scale_log2;
};
struct DecodeIO {
  float* out;
  const void* q;
  const int32_t* tables;
  const int32_t* seq_lens;
  const void* k_new;   // null: no append
  const void* v_new;
  float* part_acc;     // splits > 1 only
  float* part_mz;
};
zp_status launch_decode(const DecodeGeom& g, const DecodeIO& io, const zp_kv_pool& pool,
                        void* stream);
// Bytes of split partials a decode call needs, and the checks + launch that
// every decode entry point shares (api.cpp).
size_t decode_ws_bytes(const zp_kv_pool* pool, const zp_params* params, int32_t num_reqs,
                       int32_t splits);
zp_status decode_common(const char* name, float* out, const void* q, const void* k_new,
                        const void* v_new, const zp_kv_pool* pool,
                        const int32_t* block_tables, int32_t max_blocks,
                        const int32_t* seq_lens, int32_t num_reqs,
                        const zp_params* params, int32_t splits, void* workspace,
                        size_t workspace_bytes, void* stream);

// Timing hooks: record an event pair around kernel `kind` when enabled.
void timing_before(int kind, void* stream);
void timing_after(int kind, void* stream);

}  // namespace zp
