// The verify pass for callers that cannot allocate device memory: code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation.
// The split partials (the only scratch memory the verify kernels use) live in
// a file-scope device array instead of a caller workspace; everything else is
// vgsa_verify_attention unchanged (same validation, plan and kernels).
#include <mutex>

#include "internal.h"

namespace vgsa {
namespace {

// Largest partial buffer the entry point serves: the verify partials of
// batch 16 x 64 q-heads x 5 rows at 32768 positions take 42 MB, of batch 8 x
// 32 q-heads x 7 rows at 131088 positions 59 MB.  Each GPU the library runs
// on holds one copy for the life of the process.
constexpr size_t kScratchBytes = size_t(64) << 20;

// Host code must never pass `scratch` itself to a kernel or a copy: on the
// host the name is a stand-in, not a device address.  Its address on each
// device is looked up once (scratch_address) and used instead.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_addr[kMaxDevices];  // device address of `scratch`, per device; null until looked up
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device; looked up (with that
// device current) on the first call made on each device.
vgsa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VGSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return VGSA_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return VGSA_OK;
}

}  // namespace
}  // namespace vgsa

using namespace vgsa;

extern "C" {

size_t vgsa_noalloc_scratch_bytes(void) { return kScratchBytes; }

vgsa_status vgsa_verify_attention_noalloc(const vgsa_attn_desc* desc, const void* q,
                                          const void* k_cache, const void* v_cache,
                                          const int32_t* block_table, const int32_t* seq_lens,
                                          uint32_t collect_mask, uint64_t head_mask,
                                          vgsa_logit_layout layout, float* logits, void* out,
                                          float* lse, void* stream) {
  const size_t need = vgsa_verify_workspace_bytes(desc);
  if (need == 0)  // an invalid desc: the full call reports why, before any HIP call
    return vgsa_verify_attention(desc, q, k_cache, v_cache, block_table, seq_lens, collect_mask,
                                 head_mask, layout, logits, out, lse, nullptr, 0, stream);
  if (need > kScratchBytes) return VGSA_ERR_TOO_LARGE;
  void* ws = nullptr;
  const vgsa_status st = scratch_address(&ws);
  if (st != VGSA_OK) return st;
  return vgsa_verify_attention(desc, q, k_cache, v_cache, block_table, seq_lens, collect_mask,
                               head_mask, layout, logits, out, lse, ws, kScratchBytes, stream);
}

}  // extern "C"
