// internal.h -- declarations shared by the host and device halves of the
// ConvRot library (never installed, never seen by callers).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "layout.h"

namespace convrot {

constexpr int64_t kMaxK = 16384;           // one row = one workgroup (<= 256 lanes) of the prep kernel
constexpr int64_t kMaxRows = 16777216;     // 2^24 rows / columns

bool aligned(const void* p, size_t a);
int check_shape(int64_t rows, int64_t K, int g);
// Workspace: split-K counters (2 * kSplitCounters uint32 at offset 0) | status
// word (at CONVROT_WORKSPACE_STATUS_OFFSET) | activation INT4 image (at
// CONVROT_WORKSPACE_IMAGE_OFFSET) | activation FP6 image (M > 32, when the
// weight image has its FP6 copy) | sx | split-K partial tiles, each part
// 256-byte aligned.  K is the code width (K_rot); fp6: the FP6 part exists.
size_t workspace_image_offset();
size_t workspace_image6_offset(int64_t M, int64_t K);
size_t workspace_sx_offset(int64_t M, int64_t K, bool fp6);
size_t workspace_partial_offset(int64_t M, int64_t K, bool fp6);
size_t workspace_bytes(int64_t M, int64_t K, int64_t N, bool fp6);             // the library's plan
size_t workspace_bytes_for(int64_t M, int64_t K, bool fp6, const GemmPlan& p);  // a given plan
// Words cleared by every activation step: the counters and the status word.
constexpr int kZeroWords = 2 * kSplitCounters + 1;
// Checks of a plan given from outside (test hooks): a known block tile, M > 32,
// 1 <= splits <= min(kMaxSplits, 128-K blocks), tiles x splits at most
// kSplitCounters when split, and the FP6 tile only with fp6.  Fills *plan.
int check_forced_plan(int64_t M, int64_t K, int64_t N, int tile_m, int tile_n, int splits, bool fp6, GemmPlan* plan);

}  // namespace convrot
