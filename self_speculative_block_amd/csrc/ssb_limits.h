// Sizes shared by the kernels and the host bookkeeping of the round engine (no GPU headers, so
// that the host part also builds as a plain CPU program).
#pragma once

namespace ssb {

constexpr int kKeyChunk = 64;      // fixed key chunk of attention (absolute positions)
constexpr int kPage = 16;          // tokens per KV page
constexpr int kMaxReq = 64;        // requests per batched launch
constexpr int kMaxTasks = 64;      // attention row tasks per launch
constexpr int kTaskRows = 48;      // rows per attention task (3 MFMA row tiles)
constexpr int kMaxNormParts = 128; // per-16-column norm partials (hidden <= 2048)

}  // namespace ssb
