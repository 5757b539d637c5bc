// Query-window capture: the decode step's post-RoPE queries of every request
// that holds a query slot go to row (position mod w) of that slot's window,
// one ring per (slot, layer) ([zh] §2.2 query slots, [zh] §2.1 the last w
// queries score the cache).
//
// One workgroup per (request, layer): the q_heads x head_dim row is one
// contiguous run in both the source and the destination, copied with 16-byte
// loads and stores. HBM-bound and tiny (8 KiB per row at 32 bf16 heads of
// 128); it exists so the compression input is produced on the GPU where the
// queries are, with no host round trip.
#include <hip/hip_runtime.h>

#include "zp_device.h"
#include "zp_host.h"

namespace {

constexpr int kThreads = 256;

struct CaptureArgs {
  char* q_window;
  const char* q;
  const int32_t* slot;
  const int32_t* pos;
  int32_t L, num_slots, w, row_bytes;
};

__global__ __launch_bounds__(kThreads) void capture_kernel(CaptureArgs a) {
  const int rl = blockIdx.x;
  const int r = rl / a.L, l = rl - r * a.L;
  const int s = a.slot[r];
  const int p = a.pos[r];
  if (s < 0 || s >= a.num_slots || p < 0) return;  // no slot: nothing kept
  const int row = p % a.w;
  const char* src = a.q + static_cast<int64_t>(rl) * a.row_bytes;
  char* dst = a.q_window +
              ((static_cast<int64_t>(s) * a.L + l) * a.w + row) * a.row_bytes;
  for (int off = threadIdx.x * 16; off < a.row_bytes; off += kThreads * 16)
    *reinterpret_cast<zpd::u32x4_t*>(dst + off) =
        *reinterpret_cast<const zpd::u32x4_t*>(src + off);
}

}  // namespace

namespace zp {

zp_status launch_capture(void* q_window, const void* q, const int32_t* slot,
                         const int32_t* pos, int32_t num_reqs, int32_t layers,
                         int32_t num_slots, int32_t window, int32_t row_bytes,
                         void* stream) {
  if (row_bytes % 16) return fail(ZP_EINVAL, "capture: row of %d bytes", row_bytes);
  CaptureArgs a;
  a.q_window = static_cast<char*>(q_window);
  a.q = static_cast<const char*>(q);
  a.slot = slot;
  a.pos = pos;
  a.L = layers;
  a.num_slots = num_slots;
  a.w = window;
  a.row_bytes = row_bytes;
  const unsigned grid = static_cast<unsigned>(num_reqs) * static_cast<unsigned>(layers);
  hipLaunchKernelGGL(capture_kernel, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(ZP_EHIP, "capture kernel launch: %s", hipGetErrorString(e));
  return ZP_OK;
}

}  // namespace zp
