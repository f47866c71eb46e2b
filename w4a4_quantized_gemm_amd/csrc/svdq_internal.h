// Internal declarations shared by the host translation units of libsvdq.
// Nothing here includes HIP headers, so the validation and layout logic can
// be compiled and unit-tested by a plain C++ compiler.
#pragma once

#include <cstddef>
#include <cstdint>

#include "svdq.h"

namespace svdq {

constexpr uint32_t kMagic = 0x51445653u;  // "SVDQ" little-endian
constexpr uint32_t kVersion = 3u;
constexpr uint32_t kKnownFlags = SVDQ_F_NO_SMOOTHING | SVDQ_F_FACTORS_GIVEN | SVDQ_F_HAS_BIAS;
constexpr int kMaxRank = 128;
constexpr int kMaxDim = 65536;
constexpr int kMaxM = 1 << 22;
// The activation pass splits K into at most kMaxKParts parts, and only for
// M <= kSplitMaxM (larger M fills the chip with row blocks alone); the
// workspace holds the fp32 partial T of the parts.
constexpr int kMaxKParts = 8;
constexpr int kSplitMaxM = 16384;

// 256-byte header at offset 0 of every prepared blob.
struct BlobHeader {
  uint32_t magic;
  uint32_t version;
  int32_t fmt, K, N, rank;
  uint32_t flags;
  int32_t group;
  float alpha;
  uint32_t reserved0;
  svdq_blob_layout layout;     // 9 x uint64
  uint8_t pad[256 - 40 - sizeof(svdq_blob_layout)];
};
static_assert(sizeof(BlobHeader) == 256, "blob header must be 256 bytes");

inline int group_of(int fmt) { return fmt == SVDQ_INT4_G64_FP16 ? 64 : 32; }
// bytes of one activation/weight scale entry
inline int scale_bytes_of(int fmt) { return fmt == SVDQ_INT4_G64_FP16 ? 2 : 1; }

inline uint64_t align256(uint64_t x) { return (x + 255u) & ~uint64_t(255); }

svdq_status validate_desc(const svdq_layer_desc* d);
svdq_status validate_m(int M);
bool aligned16(const void* p);
svdq_blob_layout layout_of(const svdq_layer_desc& d);

// Activation-side buffers inside a workspace: packed codes, scales, Tb.
// The INT4 GEMM splits K over at most kGemmMaxParts parts when its
// 128 x 128 output tiles number at most kGemmSplitMaxTiles (small M, where
// the tiles alone leave most CUs idle); the workspace then holds the fp32
// partial tiles of at most kGemmSplitItems (tile, part) items.
// The FP4 GEMM likewise with at most kFp4SplitMaxTiles tiles of 256 x 256
// and kFp4SplitItems items (fp32 partial M x N planes, one per part).  Both
// fit the same 16 MiB section.
constexpr int kGemmMaxParts = 8;
constexpr int kGemmSplitMaxTiles = 128;
constexpr int kGemmSplitItems = 256;
constexpr int kGemmTile = 128;
constexpr int kFp4SplitMaxTiles = 32;
constexpr int kFp4SplitItems = 64;
constexpr int kFp4Tile = 256;
constexpr uint64_t kGemmSplitBytes = uint64_t(16) << 20;
inline bool gemm_may_split(const svdq_layer_desc& d, int M) {
  if (d.fmt == SVDQ_INT4_G64_FP16) {
    const long tiles = (static_cast<long>(M) + kGemmTile - 1) / kGemmTile * ((d.N + kGemmTile - 1) / kGemmTile);
    return tiles <= kGemmSplitMaxTiles;
  }
  const long tiles = (static_cast<long>(M) + kFp4Tile - 1) / kFp4Tile * ((d.N + kFp4Tile - 1) / kFp4Tile);
  return tiles <= kFp4SplitMaxTiles;
}

struct ActLayout {
  // required: the bytes every call needs; total adds the optional last
  // section (the split-K GEMM's partial tiles: a workspace without it runs
  // the GEMM unsplit)
  uint64_t codes, scales, tb, tpart, rowstat, fold, w4a16, ypart, required, total;
  uint64_t codes_bytes, scales_bytes, tb_bytes;
};
ActLayout act_layout(const svdq_layer_desc& d, int M);

// Weight-only (W4A16) layer for small M (at most 16 rows): the bf16 pieces
// of x_hat in MFMA A-operand order sit in the workspace, one operand plane
// (up to 8 rows) or two (up to 16 rows) of K * 64 bytes each.
constexpr int kW4A16MaxM = 16;
inline int w4a16_planes(int M) { return M <= 8 ? 1 : 2; }

}  // namespace svdq
