#!/bin/bash
cd "$GRAFT_REPO_ROOT"; mkdir -p gpurun_out/sk
echo "[step] split-K tests"
timeout -k 10 400 python3 -u -m pytest -x -q --timeout 120 --timeout-method thread tests/test_matmul_gpu.py -k "128 or split_input" > gpurun_out/sk/t2.log 2>&1; rc=$?
tail -2 gpurun_out/sk/t2.log
[ $rc -eq 0 ] || exit $rc
echo "[step] sweep"
FORMS=65,128 timeout -k 10 300 python3 -u _work/sweep_sk.py > gpurun_out/sk/sweep2.log 2>&1 || exit $?
tail -8 gpurun_out/sk/sweep2.log
echo "[step] timeline"
timeout -k 10 200 python3 -u _work/tl_sk.py 64x4096x4096 > gpurun_out/sk/tl2.log 2>&1 || exit $?
grep -v "call 20" gpurun_out/sk/tl2.log | tail -6
