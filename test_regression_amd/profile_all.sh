#!/bin/bash
# Writes the committed profile summaries (profiles/*.json, profiles/*.txt) from
# the rocprofv3 output of one profiling run of bench.py (R = repository root):
#   trace:  cd /tmp && rocprofv3 --kernel-trace --stats -f csv -d $OUT/prof_trace -o t -- python3 $R/bench.py
#   counts: cd /tmp && rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/prof_fetch -o f -- python3 $R/bench.py $SHORT
#           cd /tmp && rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/prof_write -o w -- python3 $R/bench.py $SHORT
#   mfma:   cd /tmp && rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_INSTS_VALU_MFMA_MOPS_BF16
#             SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE
#             -f csv -d $OUT/prof_mfma -o m -- python3 $R/bench.py $SHORT
# with SHORT="--steps 3 --warmup 1 --no-cpu-baseline --copy-probe-gib 1 --decode-steps 16 --no-warm-start"
# (profile_run.sh runs all four).  The headline forward is the first 4 dispatches of the bf16 CG
# kernel in a SHORT run; the dynamic-stopping forward is the first 4 dispatches of the fp32 one.
# Usage: bash test_regression_amd/profile_all.sh <rocprof output dir>   (run from the repository root)
set -euo pipefail
OUT=${1:-prof_out}
F=$OUT/prof_fetch/f_counter_collection.csv
W=$OUT/prof_write/w_counter_collection.csv
SHORT='--steps 3 --warmup 1 --no-cpu-baseline --copy-probe-gib 1 --decode-steps 16 --no-warm-start'
CMD="cd /tmp && rocprofv3 --pmc FETCH_SIZE -f csv -- python3 \$R/bench.py $SHORT ; then the same with --pmc WRITE_SIZE"
PS="python -m test_regression_amd.profile_summary traffic $F $W --copy-bytes 1073741824"
C=test_regression_amd/csrc
K2="cg_h2_kernel<128, 64, mesa::bf16_t>"
K2F="cg_h2_kernel<128, 64, float>"
$PS --kernel "$K2" --first 4 --command "$CMD; first 4 dispatches = the headline forward" \
    > profiles/cg_h2_layer_bf16_d128_T4096_traffic.json
$PS --kernel "$K2F" --first 4 --command "$CMD; first 4 dispatches = the dynamic-stopping forward" \
    > profiles/cg_h2_dynamic_f32_d128_T8192_traffic.json
$PS --kernel "chunk_states_kernel<128, 64, 4, 2, mesa::bf16_t, true>" --first 4 --command "$CMD; first 4 dispatches = the headline forward" \
    --sources $C/chunk_states.hip $C/mesa_device.h > profiles/chunk_states_layer_bf16_d128_T4096_traffic.json
$PS --kernel "chunk_states_full_kernel<64, float, true>" --first 4 --command "$CMD; first 4 dispatches = the dynamic-stopping forward" \
    --sources $C/chunk_states.hip $C/mesa_device.h > profiles/chunk_states_dynamic_f32_d128_T8192_traffic.json
$PS --kernel "decode_kernel<128, false, float>" --command "$CMD" --sources $C/decode.hip $C/mesa_device.h \
    > profiles/decode_f32_d128_N256_traffic.json
$PS --kernel "qk_preprocess_kernel<128, mesa::bf16_t, mesa::bf16_t>" --command "$CMD" \
    --sources $C/qk_preprocess.hip $C/mesa_device.h > profiles/qk_preprocess_bf16_d128_T4096_W4_traffic.json
$PS --kernel "bwd_adjoint_h2_kernel<128, 64, mesa::bf16_t>" --command "$CMD" \
    --sources $C/bwd_adjoint.hip $C/cg_core.h $C/cg_h2.h $C/persistent.h $C/mesa_device.h \
    > profiles/bwd_adjoint_layer_bf16_d128_T4096_traffic.json
$PS --kernel "bwd_kv_kernel<128, 64, mesa::bf16_t>" --command "$CMD" --sources $C/bwd_kv.hip $C/cg_h2.h $C/cg_core.h $C/persistent.h $C/mesa_device.h \
    > profiles/bwd_kv_layer_bf16_d128_T4096_traffic.json
$PS --kernel "bwd_states_kernel<128, 64, 4>" --command "$CMD" --sources $C/bwd_states.hip $C/cg_h2.h $C/cg_core.h $C/persistent.h $C/mesa_device.h \
    > profiles/bwd_states_layer_bf16_d128_T4096_traffic.json
$PS --kernel "hawk_stream_kernel<mesa::bf16_t, 8, 8>" --command "$CMD" --sources $C/hawk.hip $C/mesa_device.h \
    > profiles/hawk_stream_bf16_B8_T4096_D2048_traffic.json
M=$OUT/prof_mfma/m_counter_collection.csv
MA=$OUT/prof_mfma/m_agent_info.csv
MCMD="cd /tmp && rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE -f csv -- python3 \$R/bench.py $SHORT"
PM="python -m test_regression_amd.profile_summary mfma $M $MA"
# algorithmic flops per launch: headline 8x16x4096, d=128, C=64, k=30 (524288 token-heads):
#   CG/output k(2d^2 + 2(C+1)d + 11d) + 2d^2 + 2(C+1)d per token-head; adjoint k(...) + 2(2d^2 + 2(C+1)d);
#   dynamic 4x16x8192 (tol 1e-4): n_tok (2d^2 + 2(C+1)d) + sum_t n_t (2d^2 + 2(C+1)d + 11d) = 329013330944
$PM --kernel "$K2" --first 4 --alg-flops 825170591744 \
    --command "$MCMD; first 4 dispatches = the headline forward" > profiles/cg_h2_layer_bf16_d128_T4096_mfma.json
$PM --kernel "$K2F" --first 4 --alg-flops 329013330944 \
    --command "$MCMD; first 4 dispatches = the dynamic-stopping forward" > profiles/cg_h2_dynamic_f32_d128_T8192_mfma.json
$PM --kernel "bwd_adjoint_h2_kernel<128, 64, mesa::bf16_t>" --alg-flops 851074613248 --command "$MCMD" \
    --sources $C/bwd_adjoint.hip $C/cg_core.h $C/cg_h2.h $C/persistent.h $C/mesa_device.h \
    > profiles/bwd_adjoint_layer_bf16_d128_T4096_mfma.json
$PM --kernel "chunk_states_kernel<128, 64, 4, 2, mesa::bf16_t, true>" --first 4 --command "$MCMD; first 4 dispatches = the headline forward" \
    --sources $C/chunk_states.hip $C/mesa_device.h > profiles/chunk_states_layer_bf16_d128_T4096_mfma.json
$PM --kernel "chunk_states_full_kernel<64, float, true>" --first 4 --command "$MCMD; first 4 dispatches = the dynamic-stopping forward" \
    --sources $C/chunk_states.hip $C/mesa_device.h > profiles/chunk_states_dynamic_f32_d128_T8192_mfma.json
$PM --kernel "bwd_kv_kernel<128, 64, mesa::bf16_t>" --command "$MCMD" --sources $C/bwd_kv.hip $C/cg_h2.h $C/cg_core.h $C/persistent.h $C/mesa_device.h \
    > profiles/bwd_kv_layer_bf16_d128_T4096_mfma.json
# reverse states: 6 d^2 T flops per head (one rank-1 update for P^gx, two for M, per token)
$PM --kernel "bwd_states_kernel<128, 64, 4>" --alg-flops 51539607552 --command "$MCMD" \
    --sources $C/bwd_states.hip $C/cg_h2.h $C/cg_core.h $C/persistent.h $C/mesa_device.h \
    > profiles/bwd_states_layer_bf16_d128_T4096_mfma.json
python -m test_regression_amd.profile_summary stats $OUT/prof_trace/t_kernel_stats.csv \
    --trace $OUT/prof_trace/t_kernel_trace.csv --first-kernel "$K2" --first 13 --skip 3 \
    --command 'cd /tmp && rocprofv3 --kernel-trace --stats -f csv -d $OUT/prof_trace -o t -- python3 $R/bench.py   (R = repository root, OUT = the output directory given to profile_run.sh; default bench: headline forward 3 warmup + 10 timed steps, small workloads, forward-for-training + backward, dynamic-iteration forward, decode with warm-start runs, q/k pre-processing, Hawk scan, CPU baseline; the first 13 bf16 CG kernel dispatches are the headline forward: 3 warmup, then the 10 timed)' \
    > profiles/kernels_layer_bf16_d128_T4096_bench_stats.txt
