#!/bin/bash
set -o pipefail
cd $GRAFT_REPO_ROOT/_work/abl
for r in 1 2; do
for v in base uncondr max4 both; do
  timeout -k 5 60 ./a_$v $v 16 1 || exit $?
done
done
