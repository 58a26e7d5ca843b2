// Null device backend: accepts every job and touches no memory. Linked into
// libskv_host.so, a CPU-only build of the host runtime used to test lengths,
// page tables, crop and validation on machines without a GPU. It is never
// part of libskv.so, the GPU library.
#include "backend.h"

namespace skv {

int dev_check(const Geometry&) { return SKV_OK; }
uint64_t dev_scratch_bytes(const Geometry&) { return 0; }
int dev_init(Geometry& g) {
  g.dev = nullptr;
  return SKV_OK;
}
void dev_fini(Geometry&) {}
int dev_append(const Geometry& g, const AppendJob&) {
  ++*g.launches;
  return SKV_OK;
}
int dev_pack_qkv(const Geometry& g, const uint16_t*, uint16_t*) {
  ++*g.launches;
  return SKV_OK;
}
int dev_project(const Geometry& g, const ProjectJob&) {
  ++*g.launches;
  return SKV_OK;
}
int dev_attn_decode(const Geometry& g, const AttnJob&) {
  ++*g.launches;
  return SKV_OK;
}
int dev_decode_step(const Geometry& g, const AttnJob&, const AppendJob&) {
  ++*g.launches;
  return SKV_OK;
}
int dev_decode_step_static(const Geometry& g, const AttnJob&, const AppendJob&) {
  ++*g.launches;
  return SKV_OK;
}
int dev_attn_prefill(const Geometry& g, const AttnJob&) {
  ++*g.launches;
  return SKV_OK;
}
int dev_sync(const Geometry&) { return SKV_OK; }
int dev_set_timing(Geometry&, int) { return SKV_OK; }
int dev_collect_timing(Geometry&, skv_kernel_times* out) {
  *out = skv_kernel_times{};
  return SKV_OK;
}
const char* dev_last_error() { return ""; }
int dev_probe_stream_read(const void*, uint64_t, int, void*, double*) { return SKV_ERR_UNSUPPORTED; }
int dev_probe_mfma_bf16(void*, double*) { return SKV_ERR_UNSUPPORTED; }
int dev_probe_mfma_bf16_data(const void*, void*, double*) { return SKV_ERR_UNSUPPORTED; }
int dev_probe_launch_pattern(const void*, uint64_t, int, int, int, void*, double*, double*) {
  return SKV_ERR_UNSUPPORTED;
}

}  // namespace skv
