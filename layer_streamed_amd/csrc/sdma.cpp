#include "sdma.h"

#include <chrono>

#include <hip/hip_runtime_api.h>
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

namespace mt {

namespace {
struct Find {
  uint32_t want_bdf;
  hsa_agent_t gpu{}, cpu{};
  bool have_gpu = false, have_cpu = false;
};

hsa_status_t visit(hsa_agent_t a, void* data) {
  Find* f = static_cast<Find*>(data);
  hsa_device_type_t t;
  if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &t) != HSA_STATUS_SUCCESS) return HSA_STATUS_SUCCESS;
  if (t == HSA_DEVICE_TYPE_CPU && !f->have_cpu) {
    f->cpu = a;
    f->have_cpu = true;
  } else if (t == HSA_DEVICE_TYPE_GPU && !f->have_gpu) {
    uint32_t bdf = 0;
    hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_BDFID), &bdf);
    if (bdf == f->want_bdf) {
      f->gpu = a;
      f->have_gpu = true;
    }
  }
  return HSA_STATUS_SUCCESS;
}
}  // namespace

bool SdmaCopier::init(const char** err) {
  int dev = 0, bus = 0, device = 0, domain = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&bus, hipDeviceAttributePciBusId, dev) != hipSuccess ||
      hipDeviceGetAttribute(&device, hipDeviceAttributePciDeviceId, dev) != hipSuccess ||
      hipDeviceGetAttribute(&domain, hipDeviceAttributePciDomainID, dev) != hipSuccess) {
    *err = "cannot query the HIP device's PCI location";
    return false;
  }
  if (hsa_init() != HSA_STATUS_SUCCESS) {
    *err = "hsa_init failed";
    return false;
  }
  hsa_inited_ = true;
  Find f;
  // BDF id as ROCr reports it: bus << 8 | device << 3 | function (function 0)
  f.want_bdf = ((uint32_t)bus << 8) | ((uint32_t)device << 3);
  hsa_iterate_agents(visit, &f);
  if (!f.have_gpu) {  // fall back to the only GPU agent when the BDF does not match
    struct Any {
      hsa_agent_t gpu{};
      int n = 0;
    } any;
    hsa_iterate_agents(
        [](hsa_agent_t a, void* d) {
          hsa_device_type_t t;
          if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &t) == HSA_STATUS_SUCCESS &&
              t == HSA_DEVICE_TYPE_GPU) {
            Any* x = static_cast<Any*>(d);
            if (x->n++ == 0) x->gpu = a;
          }
          return HSA_STATUS_SUCCESS;
        },
        &any);
    if (any.n == 1) {
      f.gpu = any.gpu;
      f.have_gpu = true;
    }
  }
  if (!f.have_gpu || !f.have_cpu) {
    *err = "no matching HSA GPU/CPU agent";
    return false;
  }
  uint32_t mask = 0;
  if (hsa_amd_memory_copy_engine_status(f.cpu, f.gpu, &mask) != HSA_STATUS_SUCCESS || mask == 0) {
    *err = "no SDMA engine available for device-to-host copies";
    return false;
  }
  // ROCr's recommendation for this direction (on MI355X it names every
  // engine).  Engine 0 carries the runtime's own host-to-device copies (the
  // weight loads); sharing it serializes the two directions, so the
  // offload takes the lowest recommended engine after it (engine 1 moves
  // 57 GB/s to pinned host memory while engine 0 loads weights).
  uint32_t pref = 0;
  if (hsa_amd_memory_get_preferred_copy_engine(f.cpu, f.gpu, &pref) != HSA_STATUS_SUCCESS ||
      (pref & mask) == 0)
    pref = mask;
  pref &= mask;
  if (pref & ~1u) pref &= ~1u;
  unsigned e = 1;
  while (!(pref & e)) e <<= 1;
  hsa_signal_t sig;
  if (hsa_signal_create(1, 0, nullptr, &sig) != HSA_STATUS_SUCCESS) {
    *err = "hsa_signal_create failed";
    return false;
  }
  gpu_ = f.gpu.handle;
  cpu_ = f.cpu.handle;
  signal_ = sig.handle;
  engine_ = e;
  ok_ = true;
  return true;
}

SdmaCopier::~SdmaCopier() {
  if (signal_) hsa_signal_destroy(hsa_signal_t{signal_});
  if (hsa_inited_) hsa_shut_down();
}

bool SdmaCopier::copy_d2h(void* dst_host, const void* src_dev, size_t bytes) {
  if (!ok_ || timed_out_) return false;
  if (bytes == 0) return true;
  hsa_signal_t sig{signal_};
  hsa_signal_store_screlease(sig, 1);
  hsa_status_t st = hsa_amd_memory_async_copy_on_engine(
      dst_host, hsa_agent_t{cpu_}, src_dev, hsa_agent_t{gpu_}, bytes, 0, nullptr, sig,
      static_cast<hsa_amd_sdma_engine_id_t>(engine_), true);
  if (st != HSA_STATUS_SUCCESS) return false;
  // Bounded wait: the copy engine signals completion by decrementing the
  // signal to 0 (an error sets it negative).  A copy that has not finished
  // after COPY_TIMEOUT_S is reported as a failure, so the caller's abort
  // path returns an error instead of blocking its thread for ever.
  uint64_t freq = 0;
  if (hsa_system_get_info(HSA_SYSTEM_INFO_TIMESTAMP_FREQUENCY, &freq) != HSA_STATUS_SUCCESS ||
      freq == 0)
    freq = 1000000000ull;
  const auto t0 = std::chrono::steady_clock::now();
  for (;;) {
    const hsa_signal_value_t v = hsa_signal_wait_scacquire(
        sig, HSA_SIGNAL_CONDITION_LT, 1, freq / 10, HSA_WAIT_STATE_BLOCKED);
    if (v == 0) return true;
    if (v < 0) return false;
    const double waited =
        std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    if (waited > COPY_TIMEOUT_S) {
      timed_out_ = true;
      return false;
    }
  }
}

}  // namespace mt
