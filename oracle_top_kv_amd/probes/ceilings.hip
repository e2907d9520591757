// ceilings.hip -- measurement kernels of the benchmark (not part of the attention path): the HBM
// read rate this GPU reaches on a contiguous stream and on a gather of random 256-byte rows in
// the K / V cache layout, the two ceilings that the decode kernels' HBM fractions are set
// against, and a read-only cache scrub.  Built into libhs_probes.so; C entry points.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Contiguous read: every thread reads kPer 16-byte pieces (non-temporal loads, as the decode
// kernels read V) and folds them into one word, written out so that the loads are kept.
constexpr int kPer = 16;
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4* src, size_t n16,
                                                          uint32_t* out) {
  const size_t base = (size_t)blockIdx.x * 256 * kPer + threadIdx.x;
  u32x4 r[kPer];
#pragma unroll
  for (int i = 0; i < kPer; i++) {
    const size_t j = base + (size_t)i * 256;
    r[i] = j < n16 ? __builtin_nontemporal_load(src + j) : u32x4{0, 0, 0, 0};
  }
  u32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < kPer; i++) acc ^= r[i];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Gather of the rows a token-sparse layer reads: for each (b, u) set, the K and V rows (row_bytes
// each) of its list of positions in a [B, T, Hkv, row] cache.  A workgroup takes kRows entries of
// one set; each thread issues all of its 16-byte loads before using any.
constexpr int kRows = 128;
template <int PIECES>  // 16-byte pieces per row
__global__ __launch_bounds__(256) void row_gather_kernel(const uint8_t* K, const uint8_t* V,
                                                         const int32_t* idx, int T, int Hkv,
                                                         int cap, int chunks, uint32_t* out) {
  constexpr int kPerThread = kRows * 2 * PIECES / 256;
  const int set = blockIdx.x / chunks, ch = blockIdx.x % chunks;
  const int b = set / Hkv, u = set % Hkv;
  const int32_t* list = idx + (size_t)set * cap;
  u32x4 r[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; i++) {
    const int c = i * 256 + threadIdx.x;  // piece of the chunk: K pieces, then V pieces, per row
    const int row = c / (2 * PIECES), piece = c % (2 * PIECES);
    const int e = min(ch * kRows + row, cap - 1);
    const int pos = list[e];
    const uint8_t* base = piece < PIECES ? K : V;
    const size_t off = (((size_t)b * T + pos) * Hkv + u) * (PIECES * 16) + (piece % PIECES) * 16;
    r[i] = __builtin_nontemporal_load((const u32x4*)(base + off));
  }
  u32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < kPerThread; i++) acc ^= r[i];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

extern "C" {

// Words `out` must hold for probe_read_stream over `bytes` bytes.
size_t probe_read_stream_out_words(size_t bytes) {
  const size_t n16 = bytes / 16;
  return (n16 + 256 * kPer - 1) / (256 * kPer) * 256;
}

// Reads `bytes` (a multiple of 16) at `src`; out: probe_read_stream_out_words(bytes) words.
int probe_read_stream(const void* src, size_t bytes, uint32_t* out, void* stream) {
  const size_t n16 = bytes / 16;
  const unsigned grid = (unsigned)((n16 + 256 * kPer - 1) / (256 * kPer));
  read_stream_kernel<<<grid, 256, 0, (hipStream_t)stream>>>((const u32x4*)src, n16, out);
  return (int)hipGetLastError();
}

// Words `out` must hold for probe_row_gather.
size_t probe_row_gather_out_words(int batch, int n_kv_heads, int cap) {
  return (size_t)batch * n_kv_heads * ((cap + kRows - 1) / kRows) * 256;
}

// Gathers, for every (b, u), the K and V rows at positions idx[b, u, 0..cap-1] (each in
// [0, T)) of caches [batch, T, n_kv_heads, row_bytes]; row_bytes 256 (d 128 bf16) or 512.
int probe_row_gather(const void* k, const void* v, const int32_t* idx, int batch, int T,
                     int n_kv_heads, int cap, int row_bytes, uint32_t* out, void* stream) {
  if (batch < 1 || T < 1 || n_kv_heads < 1 || cap < 1) return (int)hipErrorInvalidValue;
  const int chunks = (cap + kRows - 1) / kRows;
  const dim3 grid((unsigned)(batch * n_kv_heads * chunks));
  if (row_bytes == 256)
    row_gather_kernel<16><<<grid, 256, 0, (hipStream_t)stream>>>(
        (const uint8_t*)k, (const uint8_t*)v, idx, T, n_kv_heads, cap, chunks, out);
  else if (row_bytes == 512)
    row_gather_kernel<32><<<grid, 256, 0, (hipStream_t)stream>>>(
        (const uint8_t*)k, (const uint8_t*)v, idx, T, n_kv_heads, cap, chunks, out);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // extern "C"
