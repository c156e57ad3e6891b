// Decode attention without a caller workspace: the arrival counters and the
// per-split (max, sum, acc) partials of the split-K decode live in one
// library-owned device array per GPU, so the call allocates nothing.  For
// callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, zero when the code object is loaded, until the
// process ends.  Host code never passes the variable's name to a kernel (on
// the host it is a stand-in, not a device address); its address on each
// device is looked up once with hipGetSymbolAddress and kept.  The decode's
// last-arriving workgroup leaves every counter it used at zero, so each
// completed call leaves the array ready for the next one; calls that overlap
// on one GPU share the array and race.

#include <mutex>

#include "cdattn.h"
#include "internal.h"

using namespace cdattn;

namespace {

static __device__ __align__(256) unsigned char scratch[CODEC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];   // address of `scratch` on each device, once looked up

// Device address of `scratch` on the device of `stream`: looked up on the
// first call for that device, with that device current, then kept.
int scratch_on(hipStream_t stream, void **ptr) {
  int dev = 0;
  int rc = stream_device(stream, &dev);
  if (rc) return rc;
  if (dev < 0 || dev >= kMaxDevices) return CODEC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return CODEC_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return CODEC_ERR_HIP;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return CODEC_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return CODEC_OK;
}

}  // namespace

extern "C" int codec_decode_attention_noalloc(const void *q, const int64_t q_stride[2], int64_t Hq,
                                              const codec_stream *k, const codec_stream *v, float scale,
                                              void *out, const int64_t out_stride[2], int32_t out_dtype,
                                              hipStream_t stream) {
  DecodePlan p;
  int rc = decode_check_args(q, q_stride, Hq, k, v, scale, out, out_stride, out_dtype, stream, &p);
  if (rc) return rc;
  // a single split writes the output directly and touches no scratch
  if (p.ns > 1 && p.bytes > (size_t)CODEC_SCRATCH_BYTES) return CODEC_ERR_WORKSPACE;
  void *ws = nullptr;
  rc = scratch_on(stream, &ws);
  if (rc) return rc;
  return launch_decode_call(q, q_stride, Hq, k, v, scale, out, out_stride, out_dtype, ws, p, nullptr, nullptr,
                            nullptr, nullptr, stream);
}
