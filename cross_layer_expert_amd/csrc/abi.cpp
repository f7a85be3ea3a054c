// Library-wide C ABI pieces: status strings, version, workspace sizing and the
// cached device properties the launchers use.
#include <hip/hip_runtime.h>

#include <atomic>

#include "cle.h"
#include "cle_internal.h"

namespace cle {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cu <= 0)
    cu = 256;
  cache[dev].store(cu, std::memory_order_relaxed);
  return cu;
}

}  // namespace cle

extern "C" const char* cle_status_string(cle_status s) {
  switch (s) {
    case CLE_OK: return "ok";
    case CLE_EINVAL: return "invalid argument";
    case CLE_EHIP: return "HIP runtime error";
    case CLE_EWORKSPACE: return "workspace missing or too small";
    case CLE_EUNSUPPORTED: return "unsupported size";
    default: return "unknown status";
  }
}

extern "C" const char* cle_version(void) { return "0.1.0"; }

static size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

extern "C" size_t cle_workspace_bytes(int32_t op, int32_t T, int32_t E, int32_t k,
                                      int32_t n_shared, int32_t n_desc) {
  if (op == CLE_OP_DISPATCH || op == CLE_OP_DISPATCH_MANY) {
    if (T < 0 || k < 1 || E < 1 || E > CLE_MAX_E) return 0;
    int64_t A = static_cast<int64_t>(T) * k;
    int64_t chunks = cle::dispatch_chunks(A);
    if (chunks < 1) chunks = 1;
    const size_t one = round_up(static_cast<size_t>(chunks) * E * sizeof(int32_t), 256);
    if (op == CLE_OP_DISPATCH) return one;
    if (n_desc < 1 || n_desc > CLE_MAX_MICROBATCHES) return 0;
    return one * static_cast<size_t>(n_desc);
  }
  if (op == CLE_OP_FFN) {
    if (E < 1 || E > CLE_MAX_E || n_shared < 0 || n_desc < 1 || n_desc > CLE_MAX_DESC) return 0;
    size_t segs = static_cast<size_t>(n_desc) * (E + n_shared);
    // header, segment table, row-tile prefix of the segments (segs + 1)
    return round_up(cle::kFfnHeader + segs * sizeof(cle::Seg) + (segs + 1) * sizeof(int32_t),
                    256);
  }
  return 0;
}
