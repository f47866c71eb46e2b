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
struct ActLayout {
  uint64_t codes, scales, tb, tpart, rowstat, fold, w4a16, total;
  uint64_t codes_bytes, scales_bytes, tb_bytes;
};
ActLayout act_layout(const svdq_layer_desc& d, int M);

// Weight-only (W4A16) layer for small M: rows are padded to kW4A16Rows[b]
// (1, 2, 4, 8 or 16), K is split into w4a16_ksplit parts (a divisor of
// K / 64) so that a part's fp32 activations fit the kernel's LDS and there
// are enough workgroups; with more than one part the fp32 partial outputs
// (parts x M x N) sit in the workspace.
constexpr int kW4A16MaxM = 16;
int w4a16_rows(int M);
int w4a16_ksplit(int M, int K, int N);

}  // namespace svdq
