// Measurement primitive: a plain streaming read of whole tiles with the
// decode kernel's load form (16-byte non-temporal buffer loads) and no
// compute.  Its rate over a random tile order is the HBM read rate a
// streaming kernel of this form reaches on the part; the decode kernel's
// achieved rate is reported against it beside the published peak.
#include <algorithm>

#include "common.h"

namespace {

using namespace pkv;

constexpr int kPiece = 4096;          // bytes one 256-lane work-group reads per load
constexpr int kPiecesInFlight = 8;    // loads issued before any is used: 32 KiB per work-group
constexpr int kReadWord3 = 0x00020000;
constexpr int kNonTemporal = 2;
constexpr uint32_t kSinkHash = 0x9E3779B9u;

struct StreamReadParams {
  const uint8_t* buf;
  const int32_t* tiles;
  uint32_t* sink;
  int64_t num_buf_tiles;   // bytes / tile_bytes
  int32_t num_tiles;
  int32_t per_wg;          // tile-list entries per work-group
  int32_t tile_bytes;
};

// Work-group b reads list entries [b * per_wg, (b + 1) * per_wg), piece by
// piece (piece p is piece p % ppt of entry p / ppt).
__global__ __launch_bounds__(256) void stream_read_kernel(StreamReadParams p) {
  const int lane = threadIdx.x;
  const int ppt = p.tile_bytes / kPiece;
  const int64_t first = (int64_t)blockIdx.x * p.per_wg;
  const int entries = (int)min((int64_t)p.per_wg, (int64_t)p.num_tiles - first);
  if (entries <= 0) return;
  const int npieces = entries * ppt;
  uint32_t acc = 0;
  for (int p0 = 0; p0 < npieces; p0 += kPiecesInFlight) {
    uint4 v[kPiecesInFlight];
#pragma unroll
    for (int j = 0; j < kPiecesInFlight; ++j) {
      const int pc = min(p0 + j, npieces - 1);   // past the end: a repeat, not used
      const int t = p.tiles[first + pc / ppt];
      const bool ok = t >= 0 && t < p.num_buf_tiles;
      const uint8_t* base = p.buf + (ok ? (int64_t)t * p.tile_bytes + (int64_t)(pc % ppt) * kPiece : 0);
      __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, ok ? kPiece : 0, kReadWord3);
      v[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, 0, kNonTemporal));
    }
#pragma unroll
    for (int j = 0; j < kPiecesInFlight; ++j)
      if (p0 + j < npieces) acc += v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  // keeps the loads live; the hash is not expected to match
  if (acc == kSinkHash) p.sink[0] = acc;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

}  // namespace

extern "C" kv_status_t kv_stream_read(const void* buf, size_t bytes, int32_t tile_bytes, const int32_t* tiles,
                                      int32_t num_tiles, uint32_t* sink, void* stream) {
  if (!buf || !tiles || !sink || num_tiles < 0 || tile_bytes < kPiece || tile_bytes % kPiece) return KV_ERR_INVALID_ARG;
  if (bytes < (size_t)tile_bytes || ((uintptr_t)buf & 15)) return KV_ERR_INVALID_ARG;
  if (num_tiles == 0) return KV_OK;
  const int cus = device_cus();
  if (cus <= 0) return KV_ERR_HIP;
  const int64_t wgs = std::min<int64_t>((int64_t)cus * 8, num_tiles);
  StreamReadParams p;
  p.buf = (const uint8_t*)buf;
  p.tiles = tiles;
  p.sink = sink;
  p.num_buf_tiles = (int64_t)(bytes / (size_t)tile_bytes);
  p.num_tiles = num_tiles;
  p.per_wg = (int32_t)((num_tiles + wgs - 1) / wgs);
  p.tile_bytes = tile_bytes;
  // entries per work-group times pieces per entry must fit an int
  if ((int64_t)p.per_wg * (tile_bytes / kPiece) > (1LL << 30)) return KV_ERR_INVALID_ARG;
  const int64_t grid = ((int64_t)num_tiles + p.per_wg - 1) / p.per_wg;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, p);
  return launch_status();
}
