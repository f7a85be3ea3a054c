// Weight packing for the grouped expert launch: a one-time re-layout of
// row-major bf16 expert weights so that every operand load of the expert
// GEMM reads 1 KiB of contiguous memory.
//
// A [R, K] matrix (R % 16 == 0, K % 64 == 0) is cut into blocks of 16 rows x
// 64 K (2 KiB), stored in (row block, K block) order.  A block is two 1 KiB
// groups (rows 0-7, rows 8-15); in a group, 16-byte chunk c (8 K elements) of
// row r sits at position r * 8 + (c ^ r): exactly where the expert launch's
// direct-to-LDS loads of a row-major matrix place it in LDS.  So a packed
// block lands in LDS byte for byte as a row-major one does, and the results
// are bitwise the same; only the global access pattern changes (one
// contiguous 1 KiB per load instruction instead of 8 rows of 128 bytes, 4 KiB
// apart, which the vector memory path serves about a third slower).
#include "cle_internal.h"

namespace cle {
namespace {

// One thread per 16-byte chunk of the packed output.
__global__ __launch_bounds__(256) void pack_kernel(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst, int64_t chunks,
                                                   int R, int K) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= chunks) return;
  const int64_t per_mat = static_cast<int64_t>(R) * K / 8;
  const int64_t mat = q / per_mat;
  const int64_t rem = q - mat * per_mat;
  const int KB = K / 64;
  const int64_t block = rem / 128;
  const int pos = static_cast<int>(rem % 128);
  const int g = pos / 64, p = pos % 64;
  const int64_t rb = block / KB;
  const int kb = static_cast<int>(block % KB);
  const int lr = p / 8, c = (p % 8) ^ lr;
  const int64_t r = rb * 16 + g * 8 + lr;
  const int64_t k = static_cast<int64_t>(kb) * 64 + c * 8;
  dst[q] = src[mat * per_mat + (r * K + k) / 8];
}

}  // namespace
}  // namespace cle

extern "C" cle_status cle_pack_weights(const void* src, void* dst, int64_t n_mat, int32_t R,
                                       int32_t K, cle_dtype dt, void* stream) {
  using namespace cle;
  if (dt != CLE_BF16 || n_mat < 0 || R < 16 || R % 16 || K < 64 || K % 64) return CLE_EINVAL;
  if (n_mat == 0) return CLE_OK;
  if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16)) return CLE_EINVAL;
  const int64_t chunks = n_mat * R * static_cast<int64_t>(K) / 8;
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  if (s0 < d0 + chunks * 16 && d0 < s0 + chunks * 16) return CLE_EINVAL;  // must not overlap
  const int64_t blocks = (chunks + 255) / 256;
  if (blocks > INT32_MAX) return CLE_EUNSUPPORTED;
  pack_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, as_stream(stream)>>>(
      static_cast<const uint4*>(src), static_cast<uint4*>(dst), chunks, R, K);
  return launch_status();
}
