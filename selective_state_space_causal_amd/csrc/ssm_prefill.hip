// ssm_prefill.hip -- choice of prefill decomposition.
#include "ssm_internal.h"

namespace ssm {

hipError_t launch_sequential(const ScanArgs& a, hipStream_t s);

int choose_prefill_variant(const ScanArgs& a) {
  (void)a;
  return kSequential;
}

size_t prefill_workspace_bytes(const ScanArgs& a) {
  (void)a;
  return 0;
}

hipError_t launch_prefill(const ScanArgs& a, void* workspace, hipStream_t s) {
  (void)workspace;
  switch (choose_prefill_variant(a)) {
    default:
      return launch_sequential(a, s);
  }
}

}  // namespace ssm
