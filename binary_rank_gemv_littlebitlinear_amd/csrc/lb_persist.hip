// Persistent whole-stack sweep (not yet available: every stack runs the
// per-layer kernels).
#include "lb_persist.h"

namespace lbi {

struct PersistPlan {};

lb_status persist_build(const std::vector<lb_layer *> &, const std::vector<int> &,
                        const std::vector<int> &, float, int, PersistPlan **out) {
  *out = nullptr;
  return LB_EUNSUPPORTED;
}
void persist_free(PersistPlan *p) { delete p; }
int64_t persist_max_rows() { return 0; }
lb_status persist_run(PersistPlan *, const uint16_t *, uint16_t *, uint16_t *const *,
                      uint16_t *const *, int64_t, hipStream_t) {
  return LB_EUNSUPPORTED;
}

}  // namespace lbi
