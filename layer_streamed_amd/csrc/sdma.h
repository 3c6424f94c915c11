// Device -> host copies on an SDMA engine through ROCr.
//
// On MI355X a copy whose writes to host memory are issued by shader code (a
// blit kernel, or any kernel storing to pinned memory) slows concurrent
// compute kernels about 2x, while the copy engines do not; hipMemcpyAsync
// may pick either for device -> host, so the gradient offload asks ROCr
// for a copy engine explicitly.
#pragma once

#include <stddef.h>

namespace mt {

class SdmaCopier {
 public:
  // Binds to the HSA agent of the current HIP device.  Returns false (and
  // a message) if ROCr or an SDMA engine is unavailable.
  bool init(const char** err);
  ~SdmaCopier();
  // Blocking copy of `bytes` from device memory to pinned host memory.
  // Returns false if the copy could not be issued, the engine reported an
  // error, or it did not finish within COPY_TIMEOUT_S; after a time-out the
  // copier refuses further copies (the engine may still hold the signal).
  bool copy_d2h(void* dst_host, const void* src_dev, size_t bytes);
  bool ready() const { return ok_ && !timed_out_; }
  static constexpr double COPY_TIMEOUT_S = 60.0;

 private:
  bool ok_ = false;
  bool hsa_inited_ = false;
  bool timed_out_ = false;
  unsigned long long gpu_ = 0, cpu_ = 0;  // hsa_agent_t handles
  unsigned long long signal_ = 0;         // hsa_signal_t handle
  unsigned engine_ = 0;
};

}  // namespace mt
