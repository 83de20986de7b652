// Probe instances of the rearrangement executors.
#include "registry.hpp"
using namespace b2bk;
#define B2B_PROBE(DT, MODE, ORN) \
    static ::b2b::ProbeRegistrar B2B_CAT(b2b_probe_, __LINE__)(::b2b::describe_probe<DT, MODE, ORN>())
B2B_PROBE(DT_F16, MODE_BPERM, false);
B2B_PROBE(DT_F16, MODE_PERMLANE, false);
B2B_PROBE(DT_F16, MODE_LDS, false);
B2B_PROBE(DT_F16, MODE_RELABEL, false);
B2B_PROBE(DT_F16, MODE_BPERM, true);
B2B_PROBE(DT_F16, MODE_LDS, true);
B2B_PROBE(DT_BF16, MODE_BPERM, false);
B2B_PROBE(DT_BF16, MODE_PERMLANE, false);
B2B_PROBE(DT_BF16, MODE_LDS, false);
B2B_PROBE(DT_BF16, MODE_RELABEL, false);
B2B_PROBE(DT_BF16, MODE_BPERM, true);
B2B_PROBE(DT_BF16, MODE_LDS, true);
B2B_PROBE(DT_F64, MODE_BPERM, false);
B2B_PROBE(DT_F64, MODE_PERMLANE, false);
B2B_PROBE(DT_F64, MODE_LDS, false);
B2B_PROBE(DT_F64, MODE_RELABEL, false);
B2B_PROBE(DT_F64, MODE_BPERM, true);
B2B_PROBE(DT_F64, MODE_LDS, true);
static ::b2b::MfmaProbeRegistrar mfma_probe_f16(::b2b::describe_mfma_probe<DT_F16>());
static ::b2b::MfmaProbeRegistrar mfma_probe_bf16(::b2b::describe_mfma_probe<DT_BF16>());
static ::b2b::MfmaProbeRegistrar mfma_probe_f64(::b2b::describe_mfma_probe<DT_F64>());
static ::b2b::MfmaProbeRegistrar mfma32_probe_f16(::b2b::describe_mfma32_probe<DT_F16>());
static ::b2b::MfmaProbeRegistrar mfma32_probe_bf16(::b2b::describe_mfma32_probe<DT_BF16>());
