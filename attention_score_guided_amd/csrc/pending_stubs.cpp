// Entry points declared in kvsel.h whose kernels are not in this build yet:
// they validate nothing and return KVSEL_ERR_UNSUPPORTED.
#include "../../include/kvsel.h"

extern "C" {

int kvsel_snapkv_vote(const kvsel_paged_kv*, const void*, int32_t, int32_t, int32_t, float, int32_t,
                      float*, int64_t, void*, size_t, void*) {
  return KVSEL_ERR_UNSUPPORTED;
}
size_t kvsel_snapkv_workspace_bytes(const kvsel_paged_kv*, int32_t, int32_t) { return 0; }

}  // extern "C"
