// internal.h -- declarations shared by the host and device halves of the
// ConvRot library (never installed, never seen by callers).
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace convrot {

constexpr int64_t kMaxK = 16384;           // one row = one workgroup (<= 256 lanes) of the prep kernel
constexpr int64_t kMaxRows = 16777216;     // 2^24 rows / columns

bool aligned(const void* p, size_t a);
int check_shape(int64_t rows, int64_t K, int g);
// Workspace: split-K counters (2 * kSplitCounters uint32 at offset 0) |
// activation INT4 image (at CONVROT_WORKSPACE_IMAGE_OFFSET) | activation FP6
// image (M > 32 only) | sx | split-K partial tiles, each part 256-byte aligned.
size_t workspace_image_offset();
size_t workspace_image6_offset(int64_t M, int64_t K);
size_t workspace_sx_offset(int64_t M, int64_t K);
size_t workspace_partial_offset(int64_t M, int64_t K);
size_t workspace_bytes(int64_t M, int64_t K, int64_t N);

}  // namespace convrot
