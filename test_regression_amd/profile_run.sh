#!/bin/bash
# The four rocprofv3 runs whose output profile_all.sh summarises (run from
# the repository root on a GPU; writes under the directory given as the
# first argument, prof_out by default).  Each pass is
# bounded by its own time limit, and the script stops at the first failure.
set -euo pipefail
R=$(pwd)
OUT=$R/${1:-prof_out}
SHORT="--steps 3 --warmup 1 --no-cpu-baseline --copy-probe-gib 1 --decode-steps 16 --no-warm-start"
mkdir -p $OUT
cd /tmp
export TMPDIR=/tmp
echo "[profile] kernel trace (default bench)"
timeout -k 10 600 rocprofv3 --kernel-trace --stats -f csv -d $OUT/prof_trace -o t -- python3 $R/bench.py > $OUT/prof_trace.log 2>&1
echo "[profile] FETCH_SIZE"
timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/prof_fetch -o f -- python3 $R/bench.py $SHORT > $OUT/prof_fetch.log 2>&1
echo "[profile] WRITE_SIZE"
timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/prof_write -o w -- python3 $R/bench.py $SHORT > $OUT/prof_write.log 2>&1
echo "[profile] MFMA / LDS counters"
timeout -s KILL 300 rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE -f csv -d $OUT/prof_mfma -o m -- python3 $R/bench.py $SHORT > $OUT/prof_mfma.log 2>&1
echo "[profile] done"
