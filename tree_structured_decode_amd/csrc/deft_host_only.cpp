// Host-only stand-ins for the HIP side of libdeft, linked only into the
// sanitizer build of the planner (deft_plan.cpp compiled with AddressSanitizer
// and UndefinedBehaviorSanitizer, no device code).  The planner's calls into
// the HIP side get fixed answers, and every entry point that needs a GPU
// fails with DEFT_ERR_UNSUPPORTED, so the planner's tests can run against
// that build on a machine without a GPU.
#include "deft_internal.h"

namespace deft {
int device_cu_count() { return 256; }   // the MI355X count
void release_upload(deft_plan*) {}      // this build never uploads
}  // namespace deft

using deft::fail;

static int no_gpu() { return fail(DEFT_ERR_UNSUPPORTED, "host-only sanitizer build: no GPU entry points"); }

extern "C" {
int deft_plan_upload(deft_plan*, const deft_attn_desc*, void*, size_t, void*) { return no_gpu(); }
int deft_partial_attention(const void*, const void*, const void*, const int32_t*, const deft_plan*,
                           const deft_attn_desc*, void*, float*, float*, int32_t, void*) {
  return no_gpu();
}
int deft_lse_merge(const deft_plan*, const deft_attn_desc*, const void*, const float*, const float*, int32_t,
                   void*, void*) {
  return no_gpu();
}
int deft_tree_attention(const void*, const void*, const void*, const int32_t*, const deft_plan*, void*,
                        const deft_attn_desc*, void*, size_t, void*) {
  return no_gpu();
}
int deft_tree_attention_fused(const void*, const void*, const void*, const int32_t*, deft_plan*, void*,
                              const deft_attn_desc*, void*, size_t, void*) {
  return no_gpu();
}
int deft_tree_attention_noalloc(const void*, const void*, const void*, const int32_t*, const deft_plan*, void*,
                                const deft_attn_desc*, void*) {
  return no_gpu();
}
int deft_plan_status(deft_plan*, void*) { return no_gpu(); }
}  // extern "C"
