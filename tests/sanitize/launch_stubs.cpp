// Stand-ins for the kernel launchers of librkv (each defined beside its
// kernels in a .hip file) in the host-only build that the sanitizer checks
// link. The host checks only take paths that launch nothing, so reaching
// any of these is itself a failure: it prints which launcher and aborts.
#include <stdio.h>
#include <stdlib.h>

#include "rkv_internal.hpp"

namespace {
[[noreturn]] void launched(const char* name) {
  fprintf(stderr, "unexpected kernel launch on the host: %s\n", name);
  abort();
}
}  // namespace

namespace rkv {
int launch_gram(const Geom&, int, const LayerPtrs&, const void*, const int32_t*, const int32_t*, float*, float*,
                int32_t*, void*, const float*) {
  launched("launch_gram");
}
int launch_score_f32(const Geom&, const LayerPtrs&, const void*, const int32_t*, const int32_t*, float*, float*,
                     float*, float*, int32_t*, void*, const float*) {
  launched("launch_score_f32");
}
int launch_redundancy(const Geom&, const int32_t*, const int32_t*, const float*, float*, void*) {
  launched("launch_redundancy");
}
int launch_select_sampled(const Geom&, const float*, const float*, const int32_t*, int, int, float, int32_t*, void*) {
  launched("launch_select_sampled");
}
int launch_select(const Geom&, const float*, const float*, const int32_t*, const float*, const int32_t*, int32_t*,
                  float*, float*, void*, const float*, const int32_t*, int) {
  launched("launch_select");
}
int launch_sentence_penalty(const float*, const int32_t*, int, int, int, float, float*, void*) {
  launched("launch_sentence_penalty");
}
int launch_compact_ids(const Geom&, const int32_t*, int32_t*, void*) { launched("launch_compact_ids"); }
int launch_decode(const Geom&, int, const LayerPtrs&, const LayerPtrs&, const void*, const int32_t*, float*, float*,
                  void*) {
  launched("launch_decode");
}
int launch_compact_holefill(const Geom&, int, const LayerPtrs&, const LayerPtrs&, const int32_t*, int32_t*, int32_t*,
                            void*) {
  launched("launch_compact_holefill");
}
int launch_compact(const Geom&, int, const LayerPtrs&, const LayerPtrs&, const int32_t*, int32_t*, void*) {
  launched("launch_compact");
}
int launch_fused_step(const Geom&, int, const LayerPtrs&, const LayerPtrs&, const void*, int32_t*, float*, float*,
                      int32_t*, int32_t*, void*, const float*, const float*, int32_t*, int) {
  launched("launch_fused_step");
}
int launch_debug_check(const Geom&, int, const LayerPtrs&, const LayerPtrs&, const void*, const int32_t*,
                       const int32_t*, uint32_t*, void*) {
  launched("launch_debug_check");
}
int scratch_workspace(void**) { launched("scratch_workspace"); }
}  // namespace rkv
